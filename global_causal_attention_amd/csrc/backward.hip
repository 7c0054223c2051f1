// Backward pass of one attention layer for gfx950: gradients of q, k, v and the gate logits of
//   y = A(q_hat, k_hat, v) * sigmoid(g),  q_hat / k_hat = RoPE(RMSNorm(q / k)),
// banded (sliding window) or full causal, GQA with 4 query heads per KV head, head dim 128.
//
// Method: ZGCM-1 zh-TW translation page, section 2.1 "Model overview" and Figure 3 (the layer's
// forward: QK-RMSNorm, partial RoPE, window or full causal attention, the sigmoid gate); section 2.2
// and section 3.1 report training throughput, i.e. forward plus this backward. The chain rule is
// taken in the usual flash-attention form: the softmax is recomputed from the forward's row
// log-sum-exp L, and with D_t = sum_d dO_t,d O_t,d the score gradient is dS = P (dP - D),
// dP = dO V^T.
//
// Kernels (one launch each, in this order):
//  1. bwd_pre   per (token, query head): dO = dy * sigmoid(g), dg = dy * y * (1 - sigmoid(g))
//               (gated layers; without a gate dO is dy and is not copied), D = sum dy * y, and a
//               16-value bf16 row (-L log2 e and -D, each split exactly into three bf16 terms)
//               that an extra matrix-core step subtracts from the scores.
//  2. bwd_q     per (sequence, KV head, 32 queries): streams K_hat/V tiles like the forward,
//               accumulates dq_hat = scale * dS K_hat and turns it into dq in its epilogue.
//  3. bwd_kv    per (sequence, KV head, 64 keys): keeps the tile's K_hat as matrix-core operands
//               in registers and its V rows in LDS, one wave per query head streams that head's
//               rows (q_hat, dO, the -L/-D row) through its own LDS buffers, accumulates
//               dV = P^T dO and dk_hat = scale * dS^T q_hat; the 4 heads' sums meet in LDS and
//               dk_hat becomes dk in the epilogue.
// The epilogues take x_hat's gradient back through RoPE (rotation by the negated angle) and
// RMSNorm (weight 1) from rows staged in LDS.
#include "zg_mfma.hpp"

namespace zg {

namespace {

constexpr int kG = 4;                    // query heads per KV head
constexpr int kNk = 64;                  // keys per tile
constexpr int kRow = 256;                // LDS bytes per staged 128-dim bf16 row
constexpr int kTileBytes = kNk * kRow;   // 16384
constexpr int kQLds = 4 * kTileBytes;    // bwd_q: two K_hat buffers, then two V buffers

// bwd_kv: per wave two buffers of (32 q_hat rows, 32 dO rows, 32 rows of 16 bf16)
constexpr int kStepQ = 32;
constexpr int kQcOff = 0;
constexpr int kDoOff = kStepQ * kRow;          // 8192
constexpr int kAuxOff = 2 * kStepQ * kRow;     // 16384
constexpr int kStepBytes = kAuxOff + kStepQ * 32;  // 17408
constexpr int kKvWaves = kG;
constexpr int kKvVTile = kKvWaves * 2 * kStepBytes;  // 139264: the tile's V rows, shared
constexpr int kKvLds = kKvVTile + kTileBytes;        // 155648
static_assert(kKvLds <= 160 * 1024, "LDS budget");
static_assert(kKvWaves * 32 * 64 * 16 <= kKvVTile, "cross-wave reduction fits the stream buffers");

// acc += A B on the matrix cores with acc held in accumulation registers (AGPRs), whatever form
// the compiler picks for the kernel's other matrix products
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8 a, const bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-byte chunk c of a staged row r lives at chunk c ^ swz(r) (as in the forward kernels).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// x = a + b + c exactly to fp32 precision, each term a bf16 value.
__device__ __forceinline__ u32x2 split3_bf16(float x) {
  const float a = bf16lo(pack_bf16(x, 0.f));
  const float r = x - a;
  const float b = bf16lo(pack_bf16(r, 0.f));
  const float c = r - b;
  return u32x2{pack_bf16(a, b), pack_bf16(c, 0.f)};
}

__device__ __forceinline__ bf16x8 ones3(bool on) {
  const __bf16 o = (__bf16)1.0f, z = (__bf16)0.0f;
  return on ? bf16x8{o, o, o, z, z, z, z, z} : bf16x8{};
}

// Raw buffer resource over `bytes` bytes from `base` (both wave-uniform); loads past the end
// return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, __builtin_amdgcn_readfirstlane((int)n), 0x00020000);
}

// One 1 KB LDS-direct load: lane l's 16 bytes at voff go to LDS address lds + 16 l.
__device__ __forceinline__ void lds_dma(uint32_t lds, uint32_t voff, __amdgpu_buffer_rsrc_t r) {
  lds_dma16(lds, voff, r, 0u);
}

__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposing read of a staged tile for an A operand whose K index runs over rows: lane gets rows
// 16 st + {4 hi .. 4 hi + 3, 8 + 4 hi .. 8 + 4 hi + 3} (the order the score layout packs its
// weights in) of dims 32 db + (lane & 31).
struct TrOffsets {
  int off[2][4];
  __device__ __forceinline__ explicit TrOffsets(int lane) {
    const int hi = lane >> 5;
    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_dch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int row = 8 * x + tr_row;
        off[x][db] = row * kRow + 16 * ((4 * db + tr_dch) ^ swz(row)) + 8 * (lane & 1);
      }
  }
  __device__ __forceinline__ bf16x8 read(const unsigned char* buf, int st, int db) const {
    const unsigned char* base = buf + st * 16 * kRow;
    const i16x4 a = lds_read_tr(base + off[0][db]);
    const i16x4 b = lds_read_tr(base + off[1][db]);
    const i16x4 both[2] = {a, b};
    return __builtin_bit_cast(bf16x8, both);
  }
};

constexpr int kStageRow = 132;  // floats per staged fp32 row: 528 bytes, rows 4 banks apart

// dx of one 128-dim row from its x_hat gradient staged in LDS (fp32 at `srow`, rotated in place)
// for x_hat = RoPE(RMSNorm(x)), weight 1, at position pos: rotate back by the negated angle, then
// dx = (dxn - xn mean(dxn . xn)) / r with r = sqrt(mean(x^2) + eps). Two adjacent lanes per row
// (half = lane & 1 holds dims 64 half .. +63; the rotated dims all lie in half 0); x and dx are bf16
// rows in global memory.
__device__ __forceinline__ void load_row_half(const uint16_t* xrow, int half, u32x4 (&xr)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) xr[i] = reinterpret_cast<const u32x4*>(xrow + 64 * half)[i];
}

__device__ __forceinline__ void dx_from_staged(float* srow, const u32x4 (&xr)[8], uint16_t* drow,
                                               int half, int64_t pos, const RopeTableH& rt,
                                               float eps) {
  const int h = rt.half;
  if (half == 0 && h > 0) {
#pragma unroll
    for (int i = 0; i < kMaxRotHalf; ++i) {
      if (i < h) {
        float c, s;
        rope_cs(pos, rt.rev[i], c, s);
        const float a = srow[i];
        const float b = srow[i + h];
        srow[i] = a * c + b * s;
        srow[i + h] = b * c - a * s;
      }
    }
  }
  float g[64], x[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(srow + 64 * half + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) g[4 * i + j] = v[j];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) unpack8(xr[i], x + 8 * i);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) ss += x[i] * x[i];
  ss += shfl_xor_f(ss, 1);
  const float inv = rsqrtf(ss * (1.0f / kHeadDim) + eps);
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) dot += g[i] * x[i];
  dot += shfl_xor_f(dot, 1);
  const float mean = dot * inv * (1.0f / kHeadDim);  // mean(dxn . xn)
  float dx[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) dx[i] = (g[i] - x[i] * inv * mean) * inv;
#pragma unroll
  for (int i = 0; i < 8; ++i) reinterpret_cast<u32x4*>(drow + 64 * half)[i] = pack8(dx + 8 * i);
}

constexpr int kQStageLds = 4 * 32 * kStageRow * 4;  // bwd_q epilogue: 32 rows per wave
// LDS of a bwd_q workgroup: the tile buffers, or the epilogue's staged rows
constexpr int kQLdsTotal = kQStageLds > kQLds ? kQStageLds : kQLds;
static_assert(2 * kQLdsTotal <= 160 * 1024, "two bwd_q workgroups per CU");
static_assert(64 * kStageRow * 4 <= kKvVTile, "bwd_kv epilogue staging fits");

}  // namespace

// ---------------------------------------------------------------------------------------------
// 1. Per (token, query head) row; 16 lanes per row, 8 dims each.
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  const int64_t n_rows = (int64_t)p.B * p.T * p.Hq;
  if (row >= n_rows) return;  // whole 16-lane groups exit together
  const int64_t off = row * kHeadDim + 8 * c;
  float y[8], dy[8];
  unpack8(*reinterpret_cast<const u32x4*>(p.out + off), y);
  unpack8(*reinterpret_cast<const u32x4*>(p.dout + off), dy);
  float dsum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) dsum = fmaf(dy[i], y[i], dsum);
  if (p.gated) {
    float g[8], dg[8], d_o[8];
    unpack8(*reinterpret_cast<const u32x4*>(p.gate + off), g);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s = 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g[i] * kLog2e));
      d_o[i] = dy[i] * s;
      dg[i] = dy[i] * y[i] * (1.0f - s);
    }
    *reinterpret_cast<u32x4*>(p.dgate + off) = pack8(dg);
    *reinterpret_cast<u32x4*>(p.dO + off) = pack8(d_o);
  }
  // without a gate dO is dy itself: the host points dO at dout
  dsum += shfl_xor_f(dsum, 1);
  dsum += shfl_xor_f(dsum, 2);
  dsum += shfl_xor_f(dsum, 4);
  dsum += shfl_xor_f(dsum, 8);
  if (c < 2) {
    const float x = (c == 0) ? -p.lse[row] * kLog2e : -dsum;
    const u32x2 s = split3_bf16(x);
    *reinterpret_cast<u32x4*>(p.aux + row * 16 + 8 * c) = u32x4{s[0], s[1], 0u, 0u};
  }
}

// ---------------------------------------------------------------------------------------------
// 2. dq_hat. Workgroup = 4 waves = (sequence, KV head, 32 queries); wave w owns query head w of the
// group. Scores are transposed as in the forward, S^T = K_hat Q^T (one query per lane), and
// dP^T = V dO^T in the same layout, so the weights dS^T pack straight into the B operand of
// dQ^T = K_hat^T dS^T. Keys stream in tiles of 64 through two K_hat and two V buffers (each wave
// loads 16 rows of both), one barrier per tile; q_hat, dO and the -L/-D row are B operands held in
// registers. At 256 VGPRs and 68 KB of LDS two workgroups share a CU, so the load and epilogue
// latencies of one overlap the other's tiles (a banded workgroup walks only 2-3 of them).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_q_kernel(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int t_idx, bh;  // the workgroups of one (sequence, KV head) together on an XCD
  xcd_pair_major(blockIdx.x, p.B * p.Hkv, p.n_qtiles, t_idx, bh);
  const int qtile = (p.window == 0) ? (p.n_qtiles - 1 - t_idx) : t_idx;  // heavy tiles first
  const int b = bh / p.Hkv;
  const int kvh = bh - b * p.Hkv;
  constexpr int MQ = 32;
  const int r0 = qtile * MQ;
  const int T = p.T;
  const int W = p.window;
  const int head = kvh * kG + (wave & 3);
  const int qbase = r0 + 32 * (wave >> 2);
  const int my_row = qbase + l32;
  const bool valid = my_row < T;

  // B operands of this lane's query: dims 16 st + 8 hi .. + 7
  bf16x8 qf[8], dof[8], auxb;
  if (valid) {
    const int64_t rq = ((int64_t)b * T + my_row) * p.Hq + head;
    const bf16x8* qs = reinterpret_cast<const bf16x8*>(p.qc + rq * kHeadDim + 8 * hi);
    const bf16x8* ds = reinterpret_cast<const bf16x8*>(p.dO + rq * kHeadDim + 8 * hi);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      qf[st] = qs[2 * st];
      dof[st] = ds[2 * st];
    }
    auxb = *reinterpret_cast<const bf16x8*>(p.aux + rq * 16 + 8 * hi);
  } else {
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      qf[st] = bf16x8{};
      dof[st] = bf16x8{};
    }
    auxb = bf16x8{};
  }
  // A operands of the extra K step: (1, 1, 1) against the -L terms (dims 0-2 of the row) for the
  // scores, against the -D terms (dims 8-10) for dP
  const bf16x8 one_l = ones3(hi == 0);
  const bf16x8 one_d = ones3(hi == 1);

  // key tiles of the workgroup
  const int q_last = min(r0 + MQ, T) - 1;
  int k_begin = 0;
  if (W > 0) k_begin = max(0, r0 - W + 1) & ~(kNk - 1);
  const int n_tiles = (q_last + 1 - k_begin + kNk - 1) / kNk;

  // tile streaming: wave w brings rows 16 w .. 16 w + 15 of the K_hat and of the V tile, 4
  // LDS-direct loads of 4 rows each
  const int wg = wave;
  const int row_bytes = p.Hkv * kHeadDim * 2;
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + (lane >> 4);
    voff[i] = (uint32_t)(row * row_bytes + 16 * ((lane & 15) ^ swz(row)));
  }
  auto dma_part = [&](int t, bool is_v) {  // tile t of K_hat or V into buffer t & 1
    const uint16_t* slab = (is_v ? p.v : p.khat) + ((int64_t)b * T * p.Hkv + kvh) * kHeadDim;
    const int row0 = k_begin + t * kNk + 16 * wg;
    const __amdgpu_buffer_rsrc_t r =
        rsrc_of(slab + (int64_t)row0 * p.Hkv * kHeadDim, (int64_t)min(16, T - row0) * row_bytes);
    const uint32_t base = (uint32_t)(uintptr_t)smem + (is_v ? 2 * kTileBytes : 0) +
                          (t & 1) * kTileBytes + 16 * wg * kRow;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma(base + 4 * i * kRow, voff[i], r);
  };
  auto dma_tile = [&](int t) {
    dma_part(t, false);
    dma_part(t, true);
  };

  int k_off[8];  // A operand of K step st: tile row l32 (+32 per key block), dims 16 st + 8 hi
#pragma unroll
  for (int st = 0; st < 8; ++st) k_off[st] = l32 * kRow + 16 * ((2 * st + hi) ^ swz(l32));
  const TrOffsets tr(lane);
  auto rd_a = [&](const unsigned char* buf, int st, int kb) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(buf + k_off[st] + kb * 32 * kRow);
  };

  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = f32x16{};

  // tile 0 goes out behind the operand loads and one wait covers both; pinning the operands after
  // it keeps the loop free of waits on them (which would also wait for the tile loads in flight)
  dma_tile(0);
  vm_wait();
#pragma unroll
  for (int st = 0; st < 8; ++st) asm volatile("" : "+v"(qf[st]), "+v"(dof[st]));
  asm volatile("" : "+v"(auxb));
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    if (j + 1 < n_tiles) dma_tile(j + 1);
    const unsigned char* kbuf = smem + (j & 1) * kTileBytes;
    const unsigned char* vbuf = smem + 2 * kTileBytes + (j & 1) * kTileBytes;
    const int kt = k_begin + j * kNk;
    const bool need_mask = (kt + kNk - 1 > qbase) || ((W > 0) && (kt < qbase + 31 - W + 1));

    // S^T and dP^T in 18 slots of two MFMAs (one per key block): slots 0-7 S over dims 16 st,
    // slot 8 subtracts L log2 e, slots 9-16 dP, slot 17 subtracts D. Slots 9-16 also turn the
    // finished scores into P = exp2(S).
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
    auto opA = [&](int k, int kb) -> bf16x8 {
      if (k < 8) return rd_a(kbuf, k, kb);
      if (k == 8) return one_l;
      if (k == 17) return one_d;
      return rd_a(vbuf, k - 9, kb);
    };
    bf16x8 ra0 = opA(0, 0);
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      // key block 0's operand was read a slot ahead; key block 1's is read now and used by the
      // slot's second MFMA
      const bf16x8 a0 = ra0, a1 = opA(k, 1);
      if (k + 1 < 18) ra0 = opA(k + 1, 0);
      const bf16x8 bq = (k < 8) ? qf[k] : (k == 8 || k == 17) ? auxb : dof[k - 9];
      if (k < 9) {
        s[0] = mfma32(a0, bq, s[0]);
        s[1] = mfma32(a1, bq, s[1]);
      } else {
        dp[0] = mfma32(a0, bq, dp[0]);
        dp[1] = mfma32(a1, bq, dp[1]);
      }
      if (k == 8 && need_mask) {
        // masked scores to -inf (P = 0); register r of key block kb is key kt + 32 kb +
        // 8 (r / 4) + 4 hi + r % 4 of this lane's query
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool ok = (key <= my_row) && (W == 0 || key > my_row - W);
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
      }
      if (k >= 9 && k < 17) {
        const int kb = (k - 9) >> 2, c = (k - 9) & 3;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s[kb][4 * c + jj] = __builtin_amdgcn_exp2f(s[kb][4 * c + jj]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // dS = P (dP - D) packed as dQ^T's B operand: pk[st] holds key step st (key block st / 2,
    // registers 8 (st % 2) .. + 7); dQ^T += K^T dS^T over 16 slots (key step st, dim block db),
    // transposing reads one slot ahead, slot (st, c) forming pair c of pk[st + 1]
    u32x4 pk[4];
    auto form = [&](int st, int c) {
      const int kb = st >> 1, r = 8 * (st & 1) + 2 * c;
      pk[st][c] = pack_bf16(s[kb][r] * dp[kb][r], s[kb][r + 1] * dp[kb][r + 1]);
    };
#pragma unroll
    for (int c = 0; c < 4; ++c) form(0, c);
    bf16x8 rt = tr.read(kbuf, 0, 0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int st = k >> 2, db = k & 3;
      const bf16x8 a = rt;
      if (k + 1 < 16) rt = tr.read(kbuf, (k + 1) >> 2, (k + 1) & 3);
      dq[db] = mfma32(a, __builtin_bit_cast(bf16x8, pk[st]), dq[db]);
      if (st < 3) form(st + 1, db);
      __builtin_amdgcn_sched_barrier(0);
    }
    vm_wait();
    __syncthreads();
  }

  // epilogue: dq_hat rows (one query per lane, 4 dims per register group) staged in the freed
  // tile buffers (the loop ended on a barrier, so no wave reads them any more; each wave reads back
  // only its own rows, in order behind its writes), then dq with two lanes per row. The raw q rows
  // the RMSNorm derivative needs are loaded first, so their latency hides behind the staging.
  const int er = lane >> 1, ehalf = lane & 1;
  const int et = qbase + er;
  const int64_t erow = (((int64_t)b * T + min(et, T - 1)) * p.Hq + head) * kHeadDim;
  u32x4 xr[8];
  load_row_half(p.q + erow, ehalf, xr);
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * kStageRow;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const f32x4 v = {dq[db][4 * rq] * p.scale, dq[db][4 * rq + 1] * p.scale,
                       dq[db][4 * rq + 2] * p.scale, dq[db][4 * rq + 3] * p.scale};
      *reinterpret_cast<f32x4*>(stage + l32 * kStageRow + 32 * db + 8 * rq + 4 * hi) = v;
    }
  if (et < T)  // both lanes of a row agree
    dx_from_staged(stage + er * kStageRow, xr, p.dq + erow, ehalf, p.pos0 + et, p.rope, p.eps);
}

// ---------------------------------------------------------------------------------------------
// 3. dv and dk_hat. Workgroup = 4 waves = (sequence, KV head, 64 keys); wave w is query head
// 4 kvh + w. Scores are kept untransposed, S = Q K_hat^T (one key per lane, 16 queries per key
// block in registers), so P and dS pack into the B operands of dV^T = dO^T P and
// dK^T = Q^T dS, whose A operands are transposing reads of the staged dO and q_hat rows.
// Each wave streams its own head's rows 32 queries at a time into two private buffers: no
// workgroup barrier until the final cross-head sum.
__global__ __launch_bounds__(kKvWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_kv_kernel(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // for full causal attention, tile 0 has the most work; the workgroups of one (sequence, KV
  // head) together on an XCD
  int ktile, bh;
  xcd_pair_major(blockIdx.x, p.B * p.Hkv, (p.T + kNk - 1) / kNk, ktile, bh);
  const int b = bh / p.Hkv;
  const int kvh = bh - b * p.Hkv;
  const int T = p.T;
  const int W = p.window;
  const int k0 = ktile * kNk;
  const int head = kvh * kG + wave;

  // queries that see a key of the tile: k0 .. min(T, k0 + 63 + W) - 1
  const int t_end = (W > 0) ? min(T, k0 + kNk - 1 + W) : T;
  const int n_steps = (t_end - k0 + kStepQ - 1) / kStepQ;

  // V rows of the tile into LDS (shared by the 4 heads; 16 rows per wave), K_hat rows as B
  // operands in registers: key k0 + 32 kb + l32, dims 16 st + 8 hi .. + 7
  {
    const int kv_row_bytes = p.Hkv * kHeadDim * 2;
    const int row0 = k0 + 16 * wave;
    const __amdgpu_buffer_rsrc_t r =
        rsrc_of(p.v + (((int64_t)b * T + row0) * p.Hkv + kvh) * kHeadDim,
                (int64_t)min(16, T - row0) * kv_row_bytes);
    const uint32_t base = (uint32_t)(uintptr_t)smem + kKvVTile + 16 * wave * kRow;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + (lane >> 4);
      lds_dma(base + 4 * i * kRow, (uint32_t)(row * kv_row_bytes + 16 * ((lane & 15) ^ swz(row))), r);
    }
  }
  bf16x8 kB[2][8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = k0 + 32 * kb + l32;
    if (key < T) {
      const int64_t r = ((int64_t)b * T + key) * p.Hkv + kvh;
      const bf16x8* ks = reinterpret_cast<const bf16x8*>(p.khat + r * kHeadDim + 8 * hi);
#pragma unroll
      for (int st = 0; st < 8; ++st) kB[kb][st] = ks[2 * st];
    } else {
#pragma unroll
      for (int st = 0; st < 8; ++st) kB[kb][st] = bf16x8{};
    }
  }
  const bf16x8 one_l = ones3(hi == 0);
  const bf16x8 one_d = ones3(hi == 1);

  // this wave's stream: rows (b, t, head) of q_hat, dO (256 bytes) and the -L/-D row (32 bytes)
  const int qrow_bytes = p.Hq * kHeadDim * 2;
  const int arow_bytes = p.Hq * 16 * 2;
  const int64_t seq_row0 = (int64_t)b * T * p.Hq + head;  // row index of (b, 0, head)
  const uint32_t wbase = (uint32_t)(uintptr_t)smem + wave * 2 * kStepBytes;
  const uint32_t avoff = (uint32_t)((lane >> 1) * arow_bytes + 16 * (lane & 1));
  auto dma_step = [&](int i) {  // queries k0 + 32 i .. + 31 into buffer i & 1
    const int t0 = k0 + kStepQ * i;
    const int n = min(kStepQ, T - t0);
    const int64_t row = seq_row0 + (int64_t)t0 * p.Hq;
    const __amdgpu_buffer_rsrc_t rq = rsrc_of(p.qc + row * kHeadDim, (int64_t)n * qrow_bytes);
    const __amdgpu_buffer_rsrc_t rd = rsrc_of(p.dO + row * kHeadDim, (int64_t)n * qrow_bytes);
    const __amdgpu_buffer_rsrc_t ra = rsrc_of(p.aux + row * 16, (int64_t)n * arow_bytes);
    const uint32_t buf = wbase + (i & 1) * kStepBytes;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = 4 * k + (lane >> 4);
      const uint32_t voff = (uint32_t)(row * qrow_bytes + 16 * ((lane & 15) ^ swz(row)));
      lds_dma(buf + kQcOff + 4 * k * kRow, voff, rq);
      lds_dma(buf + kDoOff + 4 * k * kRow, voff, rd);
    }
    lds_dma(buf + kAuxOff, avoff, ra);
  };

  int a_off[8];  // A operand of K step st: staged row l32, dims 16 st + 8 hi
#pragma unroll
  for (int st = 0; st < 8; ++st) a_off[st] = l32 * kRow + 16 * ((2 * st + hi) ^ swz(l32));
  const TrOffsets tr(lane);

  f32x16 dv[4][2], dk[4][2];  // [dim block][key block]: D[dim 32 db + ..][key 32 kb + l32]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      dv[db][kb] = f32x16{};
      dk[db][kb] = f32x16{};
    }

  const unsigned char* vtile = smem + kKvVTile;
  // the first step's rows go out behind the V rows and the K operands, one wait for all of them;
  // the K operands are pinned after it, so the loop holds no waits on them
  dma_step(0);
  vm_wait();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int st = 0; st < 8; ++st) asm volatile("" : "+v"(kB[kb][st]));
  __syncthreads();  // every wave's V rows are in LDS
  for (int i = 0; i < n_steps; ++i) {
    vm_wait();  // this step's rows are in LDS (the wave's own loads)
    if (i + 1 < n_steps) dma_step(i + 1);
    const unsigned char* buf = smem + wave * 2 * kStepBytes + (i & 1) * kStepBytes;
    const unsigned char* qbuf = buf + kQcOff;
    const unsigned char* obuf = buf + kDoOff;
    const bf16x8 auxa = *reinterpret_cast<const bf16x8*>(buf + kAuxOff + 32 * l32 + 16 * hi);
    const int t0 = k0 + kStepQ * i;
    const bool need_mask =
        (t0 < k0 + kNk - 1) || ((W > 0) && (t0 + kStepQ - 1 >= k0 + W)) || (t0 + kStepQ > T);

    // Scores and dP, 18 slots of two MFMAs (one per key block): slots 0-7 S over dims 16 st,
    // slot 8 subtracts L log2 e, slots 9-16 dP, slot 17 subtracts D. A operands are read two
    // slots ahead, the V rows (dP's B operands) likewise. Slots 9-16 also turn the finished
    // scores into P = exp2(S) and pack P as dV's B operand.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
    auto opA = [&](int k) -> bf16x8 {
      if (k < 8) return *reinterpret_cast<const bf16x8*>(qbuf + a_off[k]);
      if (k == 8 || k == 17) return auxa;
      return *reinterpret_cast<const bf16x8*>(obuf + a_off[k - 9]);
    };
    auto opV = [&](int k, int kb) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(vtile + a_off[k - 9] + kb * 32 * kRow);
    };
    u32x4 pp[2][2], ps[2][2];  // [key block][query K step]: P and dS as B operands
    bf16x8 ra[2], rv[2][2];
    ra[0] = opA(0);
    ra[1] = opA(1);
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      const bf16x8 a = ra[k & 1];
      if (k + 2 < 18) ra[k & 1] = opA(k + 2);
      bf16x8 b0, b1;
      if (k < 8) {
        b0 = kB[0][k];
        b1 = kB[1][k];
      } else if (k == 8) {
        b0 = one_l;
        b1 = one_l;
      } else if (k < 17) {
        b0 = rv[k & 1][0];
        b1 = rv[k & 1][1];
      } else {
        b0 = one_d;
        b1 = one_d;
      }
      if (k + 2 >= 9 && k + 2 <= 16) {
        rv[k & 1][0] = opV(k + 2, 0);
        rv[k & 1][1] = opV(k + 2, 1);
      }
      if (k < 9) {
        s[0] = mfma32(a, b0, s[0]);
        s[1] = mfma32(a, b1, s[1]);
      } else {
        dp[0] = mfma32(a, b0, dp[0]);
        dp[1] = mfma32(a, b1, dp[1]);
      }
      if (k == 8 && need_mask) {
        // register r of key block kb: query t0 + 8 (r / 4) + 4 hi + r % 4, key k0 + 32 kb + l32;
        // masked scores become -inf (P = 0). Rows past T were read as zeros: their dP is finite.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int key = k0 + 32 * kb + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = t0 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool ok = (key <= t) && (W == 0 || key > t - W) && (t < T);
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
        }
      }
      if (k >= 9 && k < 17) {  // 4 of the 32 weights: key block kb, registers 4 c .. 4 c + 3
        const int kb = (k - 9) >> 2, c = (k - 9) & 3;
#pragma unroll
        for (int j = 0; j < 4; ++j) s[kb][4 * c + j] = __builtin_amdgcn_exp2f(s[kb][4 * c + j]);
        pp[kb][c >> 1][2 * (c & 1)] = pack_bf16(s[kb][4 * c], s[kb][4 * c + 1]);
        pp[kb][c >> 1][2 * (c & 1) + 1] = pack_bf16(s[kb][4 * c + 2], s[kb][4 * c + 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // dV^T += dO^T P over 8 slots (dim block db, query K step st), each slot also forming 4 of
    // the dS = P (dP - D) weights; then dK^T += Q^T dS. Transposing reads two slots ahead.
    auto opT = [&](int k) { return tr.read(k < 8 ? obuf : qbuf, (k & 7) >> 2, k & 3); };
    bf16x8 rt[2];
    rt[0] = opT(0);
    rt[1] = opT(1);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int st = (k & 7) >> 2, db = k & 3;
      const bf16x8 a = rt[k & 1];
      if (k + 2 < 16) rt[k & 1] = opT(k + 2);
      if (k < 8) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          mfma_agpr(dv[db][kb], a, __builtin_bit_cast(bf16x8, pp[kb][st]));
        const int kb = k >> 2, c = k & 3;  // dS of key block kb, registers 4 c .. 4 c + 3
        ps[kb][c >> 1][2 * (c & 1)] =
            pack_bf16(s[kb][4 * c] * dp[kb][4 * c], s[kb][4 * c + 1] * dp[kb][4 * c + 1]);
        ps[kb][c >> 1][2 * (c & 1) + 1] =
            pack_bf16(s[kb][4 * c + 2] * dp[kb][4 * c + 2], s[kb][4 * c + 3] * dp[kb][4 * c + 3]);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          mfma_agpr(dk[db][kb], a, __builtin_bit_cast(bf16x8, ps[kb][st]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // the last accumulation's results are read below by register moves the compiler cannot see
  // depend on it: wait out the matrix pipeline first
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // sum over the 4 heads: each wave stores its partial sums, then reduces a quarter of them
  // (dim block `wave` of both key blocks): dv straight to memory, dk_hat staged as rows
  f32x4* red = reinterpret_cast<f32x4*>(smem);
  f32x4 dks[8];
  // the raw k rows of the epilogue's RMSNorm derivative (waves 0 and 1, two lanes per key row)
  // are loaded now, so their latency hides behind the reduction
  const int er = 32 * (wave & 1) + (lane >> 1), ehalf = lane & 1;
  const int ekey = k0 + er;
  const int64_t erow = (((int64_t)b * T + min(ekey, T - 1)) * p.Hkv + kvh) * kHeadDim;
  u32x4 xr[8];
  if (wave < 2) load_row_half(p.k + erow, ehalf, xr);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    __syncthreads();  // the buffers (or the previous round's sums) are free
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x16& a = which ? dk[db][kb] : dv[db][kb];
          red[(wave * 32 + (db * 2 + kb) * 4 + rq) * 64 + lane] =
              f32x4{a[4 * rq], a[4 * rq + 1], a[4 * rq + 2], a[4 * rq + 3]};
        }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int blk = 8 * wave + u;
      f32x4 acc = red[blk * 64 + lane];
#pragma unroll
      for (int w = 1; w < kKvWaves; ++w) acc += red[(w * 32 + blk) * 64 + lane];
      if (which) {
        dks[u] = acc * kLn2;  // scores were in log2 units
      } else {
        const int db = blk >> 3, kb = (blk >> 2) & 1, rq = blk & 3;
        const int key = k0 + 32 * kb + l32;
        if (key < T) {
          const int64_t r = (((int64_t)b * T + key) * p.Hkv + kvh) * kHeadDim + 32 * db + 8 * rq + 4 * hi;
          *reinterpret_cast<u32x2*>(p.dv + r) =
              u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
        }
      }
    }
  }
  __syncthreads();  // every wave has read its sums
  float* stage = reinterpret_cast<float*>(smem);  // [64 keys][kStageRow]
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int kb = (u >> 2) & 1, rq = u & 3;
    *reinterpret_cast<f32x4*>(stage + (32 * kb + l32) * kStageRow + 32 * wave + 8 * rq + 4 * hi) = dks[u];
  }
  __syncthreads();
  if (wave < 2 && ekey < T)  // dk: two lanes per key row, 32 rows per wave
    dx_from_staged(stage + er * kStageRow, xr, p.dk + erow, ehalf, p.pos0 + ekey, p.rope, p.eps);
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_backward(const BwdParams& p, hipStream_t s) {
  const int64_t q_rows = (int64_t)p.B * p.T * p.Hq;
  hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((q_rows + 15) / 16)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_q_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kQLdsTotal);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_q_kernel, dim3((unsigned)((int64_t)p.n_qtiles * p.B * p.Hkv)), dim3(256),
                     kQLdsTotal, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_kv_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kKvLds);
  if (e != hipSuccess) return e;
  const int64_t n_ktiles = (p.T + kNk - 1) / kNk;
  hipLaunchKernelGGL(bwd_kv_kernel, dim3((unsigned)(n_ktiles * p.B * p.Hkv)), dim3(kKvWaves * 64),
                     kKvLds, s, p);
  return hipGetLastError();
}

}  // namespace zg
