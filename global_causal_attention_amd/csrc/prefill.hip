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
#include <type_traits>

#include "zg_mfma.hpp"

namespace zg {

namespace {

constexpr int kNk = 64;                     // keys per tile
constexpr int kRow = 256;                   // LDS bytes per K or V row (unpadded, chunk-swizzled)
constexpr int kTileBytes = kNk * kRow;      // 16384
constexpr int kLdsK0 = 0;                   // two K buffers, then two V buffers
constexpr int kLdsV0 = 2 * kTileBytes;
constexpr int kQStage0 = 4 * kTileBytes;    // then per-wave q staging: 32 chunk-swizzled rows
constexpr int kQWaveBytes = 32 * kRow;
constexpr int kLdsSlots = kQStage0 + kWaves * kQWaveBytes;  // 128 KB of tiles and q rows
constexpr int kLdsBytes = kLdsSlots + 16;  // then the dynamic schedule's three claimed items

// 16-byte chunk c of a staged row r lives at chunk c ^ swz(r). Sixteen consecutive rows read at
// one logical chunk (the QK^T operand) and the four aligned rows x four adjacent chunks of a
// transposing read (the PV operand) both land on distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// RMSNorm + partial RoPE of one head row split over a lane pair (half 0: dims 0..63, half 1:
// 64..127) for 21 rotary pairs (rot_dim 42, all in half 0), in registers: the two lanes compute
// 11 and 10 of the angles, half 0 takes its partner's through one DPP exchange and rotates.
// Same arithmetic as norm_rope_row.
__device__ __forceinline__ void norm_rope_row_r42(float* x, int half, const float* __restrict__ w,
                                                  float eps, int64_t pos, const RopeTable& rt) {
  constexpr int H = 21;
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
  float cs[H], sn[H];
#pragma unroll
  for (int j = 0; j < 11; ++j) {
    const double rev = half ? rt.rev[j + 11 < H ? j + 11 : H - 1] : rt.rev[j];
    float c_, s_;
    rope_cs(pos, rev, c_, s_);
    cs[j] = c_;
    sn[j] = s_;
    if (j + 11 < H) {
      cs[j + 11] = dpp_swap_pair(c_);
      sn[j + 11] = dpp_swap_pair(s_);
    }
  }
  if (half == 0) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float a = x[i], b = x[i + H];
      x[i] = a * cs[i] - b * sn[i];
      x[i + H] = b * cs[i] + a * sn[i];
    }
  }
}


}  // namespace

// ---------------------------------------------------------------------------------------------
// K prologue: khat[b,t,h,:] = bf16(fold(RoPE(RMSNorm(k[b,t,h,:])))), packed [B, T, Hkv, 128]
// (also run on q, with Hq rows per token, where a caller wants q_hat materialised).
// Sixteen lanes per 256-byte head row, lane c holding dims 8c..8c+7, so each load or store
// instruction moves four whole rows as one contiguous kilobyte. A wave takes 8 rows per pass (two
// per 16-lane group) and strides over the rows; the next pass's rows are loaded before this pass
// is processed. RMSNorm reduces over the group with four lane exchanges. RoPE pairs (i, i + h) are
// exchanged through the wave's own LDS rows: lane c rotates pairs c and c + 16 of its group's row,
// so each lane needs only two frequencies, picked once.
constexpr int kKpRowsPerWave = 8;
constexpr int kKpStage = 68;  // floats per staged row (64 used; padded)

__global__ __launch_bounds__(256) void kprep_kernel(KPrepParams p) {
  __shared__ __attribute__((aligned(16))) float stage[4][kKpRowsPerWave][kKpStage];
  if (blockIdx.x == 0 && p.zero_words)
    for (int i = (int)threadIdx.x; i < p.n_zero_words; i += 256) p.zero_words[i] = 0u;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int c = lane & 15;
  const int Hkv = p.Hkv, T = p.T;
  const int64_t n_rows = (int64_t)p.B * T * Hkv;
  const int h = p.rope.half;
  const int rot = 2 * h;
  const bool rotates = 8 * c < rot;  // this lane holds rotated dims

  // per-lane constants: norm weights, fold factors, the lane's two rotary frequencies
  float wv[8], fv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = 8 * c + j;
    wv[j] = p.k_norm_w ? p.k_norm_w[d] : 1.0f;
    fv[j] = (d >= rot && p.fold_w) ? p.fold_scale * p.fold_w[d] : p.fold_scale;
  }
  double rev0 = 0.0, rev1 = 0.0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (c == j) {
      rev0 = p.rope.rev[j];
      rev1 = p.rope.rev[j + 16];
    }
  }

  // wave-uniform coordinates (b, t, h) of the pass's first row, advanced by a fixed stride
  const int64_t stride = (int64_t)gridDim.x * 4 * kKpRowsPerWave;
  int64_t base = ((int64_t)blockIdx.x * 4 + wave) * kKpRowsPerWave;
  if (base >= n_rows) return;
  int64_t bt0 = base / Hkv;
  int h0 = (int)(base - bt0 * Hkv);
  int64_t b0 = bt0 / T;
  int t0 = (int)(bt0 - b0 * T);
  const int64_t s_bt = stride / Hkv;
  const int s_h = (int)(stride - s_bt * Hkv);
  const int64_t s_b = s_bt / T;
  const int s_t = (int)(s_bt - s_b * T);

  // row r of the pass (r = grp + 4 i) -> source offset, output row, position
  struct RowAt {
    int64_t src, orow, pos;
    bool valid;
  };
  auto row_at = [&](int64_t bse, int64_t b_, int t_, int h_, int r) -> RowAt {
    int hh = h_ + r;
    int tt = t_;
    int64_t bb = b_;
    while (hh >= Hkv) { hh -= Hkv; ++tt; }
    while (tt >= T) { tt -= T; ++bb; }
    RowAt o;
    o.valid = bse + r < n_rows;
    o.src = (bb * T + tt) * p.sk + (int64_t)hh * kHeadDim + 8 * c;
    o.orow = (bb * p.out_rows + p.out_row0 + tt) * Hkv + hh;
    o.pos = p.pos0 + tt;
    return o;
  };
  auto load = [&](const RowAt& ra) -> u32x4 {
    return ra.valid ? *reinterpret_cast<const u32x4*>(p.k + ra.src) : u32x4{0u, 0u, 0u, 0u};
  };

  RowAt cur[2];
  u32x4 raw[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    cur[i] = row_at(base, b0, t0, h0, grp + 4 * i);
    raw[i] = load(cur[i]);
  }
  float* st = &stage[wave][0][0];
  while (true) {
    // next pass: coordinates and loads go out before this pass is processed
    const int64_t nbase = base + stride;
    const bool more = nbase < n_rows;
    h0 += s_h;
    t0 += s_t;
    b0 += s_b;
    if (h0 >= Hkv) { h0 -= Hkv; ++t0; }
    if (t0 >= T) { t0 -= T; ++b0; }
    RowAt nxt[2];
    u32x4 nraw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      nxt[i] = row_at(nbase, b0, t0, h0, grp + 4 * i);
      nraw[i] = more ? load(nxt[i]) : u32x4{0u, 0u, 0u, 0u};
    }

    float x[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      unpack8(raw[i], x[i]);
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += x[i][j] * x[i][j];
      ss += shfl_xor_f(ss, 1);
      ss += shfl_xor_f(ss, 2);
      ss += shfl_xor_f(ss, 4);
      ss += shfl_xor_f(ss, 8);
      const float inv = rsqrtf(ss * (1.0f / kHeadDim) + p.eps);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] *= inv * wv[j];
    }
    if (h > 0) {
      // stage the rotated dims of both rows, rotate pairs c and c + 16, read back
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float* sr = st + (grp + 4 * i) * kKpStage + 8 * c;
        if (rotates) {
          *reinterpret_cast<f32x4*>(sr) = f32x4{x[i][0], x[i][1], x[i][2], x[i][3]};
          *reinterpret_cast<f32x4*>(sr + 4) = f32x4{x[i][4], x[i][5], x[i][6], x[i][7]};
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS ops complete in order
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float* sr = st + (grp + 4 * i) * kKpStage;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int pi = c + 16 * k;
          if (pi < h) {
            float cs, sn;
            rope_cs(cur[i].pos, k ? rev1 : rev0, cs, sn);
            const float a = sr[pi];
            const float b = sr[pi + h];
            sr[pi] = a * cs - b * sn;
            sr[pi + h] = b * cs + a * sn;
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float* sr = st + (grp + 4 * i) * kKpStage + 8 * c;
        if (rotates) {
          const f32x4 lo = *reinterpret_cast<const f32x4*>(sr);
          const f32x4 hi4 = *reinterpret_cast<const f32x4*>(sr + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[i][j] = lo[j];
            x[i][4 + j] = hi4[j];
          }
        }
      }
      // the next pass rewrites these rows: its writes must not overtake this pass's reads
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (p.ring_k && cur[i].valid && cur[i].pos - p.pos0 >= p.ring_t0) {
        // (b, t, h) of the row from its output row and position
        const int64_t tt = cur[i].pos - p.pos0;
        const int64_t hh = cur[i].orow % Hkv;
        const int64_t bb = (cur[i].orow / Hkv - p.out_row0 - tt) / p.out_rows;
        const int64_t rr = (bb * p.ring_w + cur[i].pos % p.ring_w) * Hkv + hh;
        *reinterpret_cast<u32x4*>(p.ring_k + rr * kHeadDim + 8 * c) = pack8(x[i]);
        *reinterpret_cast<u32x4*>(p.ring_v + rr * kHeadDim + 8 * c) = *reinterpret_cast<const u32x4*>(
            p.ring_v_src + (bb * T + tt) * p.ring_sv + hh * kHeadDim + 8 * c);
      }
      if (p.fold) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] *= fv[j];
      }
      if (cur[i].valid)
        *reinterpret_cast<u32x4*>(p.khat + cur[i].orow * kHeadDim + 8 * c) = pack8(x[i]);
    }
    if (!more) break;
    base = nbase;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      cur[i] = nxt[i];
      raw[i] = nraw[i];
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <int G, bool GATED>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  constexpr int QB = kWaves / G;   // 32-query blocks per head
  constexpr int MQ = 32 * QB;      // queries per tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform

  // ---- work items: heavy query tiles first for full causal attention, the workgroups of one
  // (sequence, KV head) together on an XCD. One item per workgroup, or (p.persist) one workgroup
  // per CU walking the items the hardware order would give its XCD, 8 * round + the CU's place in
  // the XCD, the places snaking from round to round so that every CU sees heavy and light items.
  // A persistent workgroup brings the next item's q rows into its staging rows during iteration 1
  // of the current item, and the next item's first two K tiles once the current item's last
  // iteration has read its K buffers, so neither waits on memory at the next item's start.
  // With item counters (p.counters) the schedule is dynamic: items are handed out one at a time
  // to whichever workgroup asks next (see claim below), so XCDs that run slower than others do
  // not hold up the end of the launch. Thread 0 claims
  // each item two items ahead into a ring of three LDS slots, so every wave reads an item's slot
  // at least one workgroup barrier after it was written and before it is written again.
  int item_k = 0;
  int vb = p.persist ? -1 : (int)blockIdx.x;   // -1: the schedule's first item, looked up below
  bool q_ready = false;   // this item's raw q rows are already in the staging rows
  bool k_ready = false;   // this item's first K tiles were issued during the previous item
  int* const slots = reinterpret_cast<int*>(smem + kLdsSlots);
  // Item (pair, t) -- t = 0 the pair's heaviest query tile -- is item number
  // (pair & 7) + 8 ((pair >> 3) n_qt + t) of the static order. XCD x has two queues (counters x
  // and 8 + x): the heavy three quarters (t < n_qt - n_qt / 4) of its pairs' tiles, pair by pair,
  // and the light quarter, heaviest first across its pairs. A workgroup takes from its XCD's heavy
  // queue, then from its light queue (those pairs' keys were just streamed through the XCD's L2),
  // then from the light queue whose next item is heaviest, so the launch ends on the lightest
  // items wherever they are; last from what is left in other XCDs' heavy queues.
  auto claim = [](uint32_t* ctr, int n_qt, int n_pairs) -> int {
    const int x = (int)(blockIdx.x & 7);  // workgroup i runs on XCD i mod 8
    const int n_light = n_qt >> 2, n_heavy = n_qt - n_light;
    const int ppx = n_pairs >> 3;          // pairs per XCD
    const int n_own = ppx * n_heavy;       // items per heavy queue
    const int n_lown = ppx * n_light;      // items per light queue
    auto take = [&](int q) {
      return (int)__hip_atomic_fetch_add(ctr + kSchedStride * q, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    };
    auto heavy_item = [&](int xq, int j) {
      const int pl = j / n_heavy;
      return xq + 8 * (pl * n_qt + (j - pl * n_heavy));
    };
    auto light_item = [&](int xq, int g) {
      const int tq = g / ppx;
      return xq + 8 * ((g - tq * ppx) * n_qt + n_heavy + tq);
    };
    int j = take(x);
    if (j < n_own) return heavy_item(x, j);
    int g = take(8 + x);
    if (g < n_lown) return light_item(x, g);
    // every light queue runs heaviest first, so the one with the fewest items taken has the
    // heaviest next item; a take that finds its queue empty leaves that queue out of every later
    // scan, so the loop ends within eight rounds
#pragma unroll 1
    for (int tries = 0; tries < 8; ++tries) {
      int best = -1, best_n = n_lown;
#pragma unroll 1
      for (int xs = 0; xs < 8; ++xs) {
        const int c = (int)__hip_atomic_load(ctr + kSchedStride * (8 + xs), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        if (c < best_n) {
          best_n = c;
          best = xs;
        }
      }
      if (best < 0) break;
      g = take(8 + best);
      if (g < n_lown) return light_item(best, g);
    }
#pragma unroll 1
    for (int sx = 1; sx < 8; ++sx) {
      const int xs = (x + sx) & 7;
      j = take(xs);
      if (j < n_own) return heavy_item(xs, j);
    }
    return n_qt * n_pairs;
  };
  const bool dyn = p.persist && p.counters;
  if (dyn) {
    if (tid == 0) {
      slots[0] = claim(p.counters, p.n_qtiles, p.B * p.Hkv);
      slots[1] = claim(p.counters, p.n_qtiles, p.B * p.Hkv);
    }
    __syncthreads();
  }
  while (true) {
  // The kernel arguments are read through a pointer the compiler must treat as new on every item,
  // so it loads them where the item needs them instead of keeping all of them live across the
  // loop (which would spill).
  typedef __attribute__((address_space(4))) const PrefillParams* karg_prefill_ptr;
  karg_prefill_ptr kpp = (karg_prefill_ptr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kpp));
  const __attribute__((address_space(4))) PrefillParams& p = *kpp;
  // likewise the lane index, so the per-lane offsets derived from it are recomputed per item
  // rather than held in registers through the q prologue
  int lane = tid & 63;
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_items = p.n_qtiles * p.B * p.Hkv;
  auto item_at = [&](int k) -> int {
    if (!p.persist) return k == 0 ? (int)blockIdx.x : n_items;
    const int cx = (int)(gridDim.x >> 3), x = (int)(blockIdx.x & 7), cw = (int)(blockIdx.x >> 3);
    const int cc = (k & 1) ? (cx - 1 - cw) : cw;
    const int64_t vb_ = x + 8 * ((int64_t)k * cx + cc);
    return vb_ < n_items ? (int)vb_ : n_items;
  };
  const int T = p.T;
  const int W = p.window;
  const int qoff = p.qoff;
  const bool v_loader = wave >= 4;
  const int wg = wave & 3;
  const int row_bytes = (int)((v_loader ? p.sv : (int64_t)p.Hkv * kHeadDim) * 2);
  const int q_row_bytes = (int)(p.sq * 2);
  unsigned char* qs = smem + kQStage0 + wave * kQWaveBytes;
  // key tile range of an item (key rows; query row t is key row qoff + t)
  auto item_k_begin = [&](int r0_) -> int {
    return W > 0 ? (max(0, qoff + r0_ - W + 1) & ~(kNk - 1)) : 0;
  };
  auto item_n_tiles = [&](int r0_) -> int {
    const int q_last_ = qoff + min(r0_ + MQ, T) - 1;
    return (q_last_ + 1 - item_k_begin(r0_) + kNk - 1) / kNk;
  };
  auto item_coords = [&](int vb_, int& qtile_, int& b_, int& kvh_) {
    int t_, bh_;
    xcd_pair_major(vb_, p.B * p.Hkv, p.n_qtiles, t_, bh_);
    qtile_ = (W == 0) ? (p.n_qtiles - 1 - t_) : t_;
    b_ = bh_ / p.Hkv;
    kvh_ = bh_ - b_ * p.Hkv;
  };
  auto kv_rsrc = [&](int b_, int kvh_) {
    const uint16_t* slab_ = v_loader ? p.v + (int64_t)b_ * p.kv_rows * p.sv + (int64_t)kvh_ * kHeadDim
                                     : p.khat + ((int64_t)b_ * p.kv_rows * p.Hkv + kvh_) * kHeadDim;
    return __builtin_amdgcn_make_buffer_rsrc((void*)slab_, 0,
                                             (int)((uint32_t)p.n_keys * (uint32_t)row_bytes),
                                             0x00020000);  // byte count < 2^32, read as unsigned
  };
  // lane -> (row (lane >> 4) of the 4-row group i, physical chunk lane & 15)
  auto dma_voff = [&](int i) -> uint32_t {
    const int row = 4 * i + (lane >> 4);  // row within the wave's 16 (swizzle uses row & 15)
    return (uint32_t)((lane >> 4) * row_bytes + 16 * ((lane & 15) ^ swz(row)));
  };
  const uint32_t lds_k = (uint32_t)(uintptr_t)smem + kLdsK0;
  const uint32_t lds_v = (uint32_t)(uintptr_t)smem + kLdsV0;
  // tile t of the keys starting at key row kb0 into buffer t & 1
  auto dma_tile_at = [&](__amdgpu_buffer_rsrc_t rs_, int kb0, int t, bool is_v) {
    const uint32_t base = (is_v ? lds_v : lds_k) + (t & 1) * kTileBytes + 16 * wg * kRow;
    const uint32_t row0 = (uint32_t)(kb0 + t * kNk + 16 * wg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m0v = base + 4 * i * kRow;
      const uint32_t soff = (row0 + 4 * i) * (uint32_t)row_bytes;
      lds_dma16(m0v, dma_voff(i), rs_, soff);
    }
  };
  // this wave's 32 raw q rows of an item into its staging rows (row r at r * kRow, chunk c at
  // c ^ swz(r)): 8 instructions of 4 rows; rows at or past T read as zeros
  auto dma_q_rows = [&](int b_, int head_, int row0_) {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.q + (int64_t)b_ * T * p.sq + (int64_t)head_ * kHeadDim), 0,
        (int)((uint32_t)T * (uint32_t)q_row_bytes), 0x00020000);
    const uint32_t lq = (uint32_t)(uintptr_t)qs;
    // the rows' previous contents (the current item's operands) have been read out
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      const uint32_t voff = (uint32_t)((lane >> 4) * q_row_bytes + 16 * ((lane & 15) ^ swz(r)));
      lds_dma16(lq + i * 1024, voff, rq, (uint32_t)(row0_ + 4 * i) * (uint32_t)q_row_bytes);
    }
  };
  auto vm_wait = []() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  const int hg = wave % G;
  const int qb = wave / G;
  const float c = p.scale_log2;

  if (dyn) vb = __builtin_amdgcn_readfirstlane(slots[item_k % 3]);
  else if (vb < 0) vb = item_at(0);
  if (vb >= n_items) break;
  const int vb_next =
      dyn ? __builtin_amdgcn_readfirstlane(slots[(item_k + 1) % 3]) : item_at(item_k + 1);
  if (dyn && tid == 0) slots[(item_k + 2) % 3] = claim(p.counters, p.n_qtiles, p.B * p.Hkv);
  const bool has_next = vb_next < n_items;
  int qtile, b, kvh;
  item_coords(vb, qtile, b, kvh);
  const int r0 = qtile * MQ;
  const int head = kvh * G + hg;
  const int qbase = r0 + 32 * qb;
  const int k_begin = item_k_begin(r0);
  const int n_tiles = item_n_tiles(r0);
  // the next item's q rows come into the staging rows as soon as this item's prologue has read
  // them (the register RoPE of 42 dims keeps the staging rows free of scratch)
  const bool prefetch_q = p.persist && has_next && p.rope.half == 21;

  // ---- tile streaming: waves 0-3 bring K rows, waves 4-7 V rows, straight into chunk-swizzled
  // LDS rows (buffer_load ... lds, 4 rows = 1 KB per instruction, 4 per wave per tile). The
  // buffer's range check returns zeros for rows at or past T. Iteration j reads K_{j+1} and V_{j-1}
  // and streams K_{j+2} and V_j into the buffers those tiles' predecessors left; the loads are
  // inline asm (so later LDS reads do not wait for them) and are awaited before the barrier that
  // ends the iteration.
  const __amdgpu_buffer_rsrc_t rsrc = kv_rsrc(b, kvh);
  auto dma_tile = [&](int t, bool is_v) { dma_tile_at(rsrc, k_begin, t, is_v); };

  // the first two K tiles go out before the q prologue (unless the previous item issued them)
  if (!v_loader && !k_ready) {
    dma_tile(0, false);
    if (n_tiles > 1) dma_tile(1, false);
  }

  // ---- q prologue: q_hat * scale * log2(e) rounded to bf16, staged through this wave's own
  // chunk-swizzled rows and read back as MFMA B operands. It runs while the first two K tiles
  // are in flight.
  bf16x8 qf[8];
  {
    const int r = lane >> 1;
    const int half = lane & 1;
    const int t = qbase + r;
    float x[64];
    if (q_ready) {
      // prefetched raw rows (landed: iteration 2 of the previous item waited for them)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        unpack8(*reinterpret_cast<const u32x4*>(qs + r * kRow + 16 * ((8 * half + i) ^ swz(r))),
                x + 8 * i);
      // every lane has read its half row before any lane of the wave writes q_hat over it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else if (t < T) {
      const u32x4* s4 = reinterpret_cast<const u32x4*>(
          p.q + ((int64_t)b * T + t) * p.sq + (int64_t)head * kHeadDim + 64 * half);
#pragma unroll
      for (int i = 0; i < 8; ++i) unpack8(s4[i], x + 8 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = 0.f;
    }
    if (p.rope.half == 21) {
      norm_rope_row_r42(x, half, p.q_norm_w, p.eps, p.pos0 + t, *(const RopeTableH*)&p.rope);
    } else {
      // the [dim][row] RoPE scratch (32 rows x 64 floats) overlays this wave's staging rows;
      // every access to it precedes the bf16 row writes below in this wave's program order
      norm_rope_row(x, half, p.q_norm_w, p.eps, p.pos0 + t, *(const RopeTableH*)&p.rope,
                    reinterpret_cast<float*>(qs),
                    r, 32);
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] *= c;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(qs + r * kRow + 16 * ((8 * half + i) ^ swz(r))) = pack8(x + 8 * i);
    // the wave reads back only its own rows, and its LDS operations complete in order
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(qs + l32 * kRow + 16 * ((2 * s + hi) ^ swz(l32)));
  }


  // ---- MFMA operand addresses: per-lane byte offsets, everything else is an immediate
  int k_off[8];     // QK^T operand of step st: key row l32 (+32 per key block), dims 16 st + 8 hi
#pragma unroll
  for (int st = 0; st < 8; ++st) k_off[st] = kLdsK0 + l32 * kRow + 16 * ((2 * st + hi) ^ swz(l32));
  int v_off[2][4];  // PV operand, transposing read x of dim block db (+16 rows per key step)
  {
    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_dch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int row = 8 * x + tr_row;
        v_off[x][db] = kLdsV0 + row * kRow + 16 * ((4 * db + tr_dch) ^ swz(row)) + 8 * (lane & 1);
      }
  }
  // 9th key-dimension step: A = (1, 0, ...) on every key row, B = (-m_ref, 0, ...) per query, so
  // the MFMA subtracts the softmax reference and exp2 needs no extra arithmetic
  const bf16x8 one_op = hi ? bf16x8{} : bf16x8{(__bf16)1.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f,
                                               (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
  float m_ref = 0.f;          // bf16-representable softmax reference (log2 units), per query
  bool m_valid = false;       // set once the query has seen an unmasked key
  bf16x8 qm = bf16x8{};       // B operand of the 9th step
  // The reference is free as long as exp2 stays in range: it is 0 unless the first tile's maximum
  // lies outside [-32, 32] or a later tile forces a rescale, and while it is 0 on every lane of
  // the wave the 9th step would add zero and is skipped.
  bool need_ref = false;      // wave-uniform

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float l_run = 0.f;
  const int my_row = qbase + l32;   // query row
  const int my_q = qoff + my_row;   // its key row
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  auto rd_k = [&](int par, int st, int kb) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(smem + k_off[st] + par * kTileBytes + kb * 32 * kRow);
  };
  auto rd_v = [&](int par, int st, int db) -> bf16x8 {
    const unsigned char* base = smem + par * kTileBytes + st * 16 * kRow;
    const i16x4 a = lds_read_tr(base + v_off[0][db]);
    const i16x4 bb = lds_read_tr(base + v_off[1][db]);
    const i16x4 both[2] = {a, bb};
    return __builtin_bit_cast(bf16x8, both);
  };
  auto qk_all = [&](int par, f32x16 (&s)[2]) {  // S = K Q^T - m_ref, all 18 MFMAs
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(rd_k(par, st, kb), qf[st], s[kb]);
    if (need_ref) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(one_op, qm, s[kb]);
    }
  };
  auto mask_tile = [&](int j, f32x16 (&s)[2]) {
    const int kt = k_begin + j * kNk;
    const bool need = (kt + kNk - 1 > qoff + qbase) || ((W > 0) && (kt < qoff + qbase + 31 - W + 1));
    if (need) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = (key <= my_q) && (W == 0 || key > my_q - W);
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
    }
  };
  // Softmax weights of the current tile: P = exp2(S) (S already has the reference subtracted).
  // Unless a lane's tile sum exceeds 2^64 (or the query has no reference yet) nothing needs
  // rescaling; otherwise the slow path sets the reference (0 for a first tile whose maximum lies
  // in [-32, 32], else the running maximum), rescales l and O, redoes P, and moves the already
  // computed next-tile scores to the new reference.
  auto slow_path = [&](f32x16 (&s)[2], f32x16 (&sn)[2], u32x4 (&pk)[4], float& rs) {
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = fmaxf(mx, __uint_as_float(hi ? sw[0] : sw[1])) + m_ref;  // tile maximum, log2 units
    const bool has = mx > -INFINITY;
    float m_new = m_valid ? fmaxf(m_ref, mx) : (fabsf(mx) <= 32.f ? 0.f : mx);
    m_new = has || m_valid ? bf16lo(pack_bf16(m_new, 0.f)) : m_ref;
    const float alpha = m_valid ? __builtin_amdgcn_exp2f(m_ref - m_new) : 0.f;
    const float delta = m_ref - m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= alpha;
    float part = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[kb][r] + delta);
        const float p1 = __builtin_amdgcn_exp2f(s[kb][r + 1] + delta);
        const uint32_t w = pack_bf16(p0, p1);
        pk[2 * kb + (r >> 3)][(r >> 1) & 3] = w;
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, part, false);
      }
    rs = part;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[kb][r] += delta;
    m_ref = m_new;
    m_valid = m_valid || has;
    qm = hi ? bf16x8{} : bf16x8{(__bf16)(-m_new), (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f,
                                (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
    need_ref = __builtin_amdgcn_ballot_w64(m_ref != 0.f) != 0;
  };

  // One iteration j >= 1 (buffer parity PAR = j & 1): 32 MFMAs (34 with the 9th step) issued one
  // by one, each followed by a slice of tile j's softmax (an exponential, plus a pack and a
  // row-sum step every other slot), which runs in the MFMA shadow. The slots:
  //   0-1    the last key-dimension step of S_j (K_j, read before the previous barrier)
  //   2-17   PV of tile j-1 with its weights
  //   18-31  QK^T of tile j+1, key-dimension steps 0-6 (step 7 opens the next iteration)
  // The A operands stream through a two-deep ring that runs on across iterations: the last two
  // reads of an iteration fetch the next one's slots 0-1 from K_{j+1}, which every wave can
  // already see, so after the barrier the matrix work resumes without waiting on LDS. Masking
  // S_j before its last step is exact (a -inf partial sum stays -inf), and so is the slow path's
  // shift of the partial S_{j+1} (the remaining step adds on top of it).
  constexpr int kAhead = 2;
  bf16x8 ring[kAhead];
  auto iter = [&](int j, auto par_c, f32x16 (&sc)[2], f32x16 (&sn)[2], u32x4 (&pk_prev)[4],
                  u32x4 (&pk_cur)[4]) {
    constexpr int PAR = decltype(par_c)::value;
    mask_tile(j, sc);
    float e[32];
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sn[kb] = f32x16{};
    // A operand of slot i; slots 32 and 33 are the next iteration's slots 0 and 1
    auto opnd = [&](int i) -> bf16x8 {
      if (i < 2) return rd_k(PAR, 7, i);
      if (i < 18) return rd_v(PAR ^ 1, (i - 2) >> 2, (i - 2) & 3);
      if (i < 32) return rd_k(PAR ^ 1, (i - 18) >> 1, (i - 18) & 1);
      return rd_k(PAR ^ 1, 7, i - 32);
    };
    // one exponential of tile j's scores, and the pack and row-sum step of each completed pair
    auto soft = [&](int k) {
      e[k] = __builtin_amdgcn_exp2f(sc[k >> 4][k & 15]);
      if (k & 1) {
        const int pr = k >> 1;
        uint32_t w = pack_bf16(e[k - 1], e[k]);
        float ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones,
                                                   part[pr & 3], false);
        // pins the pair's work to this slot: the compiler would otherwise sink it past the
        // branch around the 9th step, out of the MFMA shadow
        asm volatile("" : "+v"(w), "+v"(ps));
        pk_cur[pr >> 2][pr & 3] = w;
        part[pr & 3] = ps;
      }
    };
#pragma unroll
    for (int i = 0; i < 34; ++i) {
      // matrix work
      if (i < 32) {
        const bf16x8 a = ring[i % kAhead];
        ring[i % kAhead] = opnd(i + kAhead);
        if (i < 2) {
          sc[i] = mfma32(a, qf[7], sc[i]);
        } else if (i < 18) {
          const int st = (i - 2) >> 2, db = (i - 2) & 3;
          o[db] = mfma32(a, __builtin_bit_cast(bf16x8, pk_prev[st]), o[db]);
        } else {
          const int st = (i - 18) >> 1, kb = (i - 18) & 1;
          sn[kb] = mfma32(a, qf[st], sn[kb]);
        }
      } else {
        const int kb = i - 32;
        if (need_ref) sn[kb] = mfma32(one_op, qm, sn[kb]);
      }
      if (i == 1) {
        // the buffers these tiles go to were last read before the barrier that opened this
        // iteration
        if (v_loader) dma_tile(j, true);
        else if (j + 2 < n_tiles) dma_tile(j + 2, false);
      }
      // vector work on tile j's scores, from slot 2 on (S_j is complete after slots 0-1)
      if (i >= 2 && i < 32) soft(i - 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    soft(30);
    soft(31);
    float rs = (part[0] + part[1]) + (part[2] + part[3]);
    if (__builtin_amdgcn_ballot_w64(!m_valid || !(rs <= 0x1p64f))) slow_path(sc, sn, pk_cur, rs);
    l_run += rs;
    vm_wait();  // this iteration's tiles have landed
    __syncthreads();
  };

  // the next item's raw q rows (the prologue above has read this item's out of the staging rows);
  // they are the last 8 loads issued, so the preamble waits for everything before them
  if (prefetch_q) {
    int qt_n, b_n, kvh_n;
    item_coords(vb_next, qt_n, b_n, kvh_n);
    dma_q_rows(b_n, kvh_n * G + hg, qt_n * MQ + 32 * qb);
  }

  // ---- preamble: K_0 and K_1 in LDS, S_0 computed
  if (prefetch_q) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else vm_wait();
  __syncthreads();
  f32x16 sA[2], sB[2];
  u32x4 pA[4], pB[4];
  qk_all(0, sA);
  __syncthreads();  // K_0's buffer is refilled during iteration 0
  // iteration 0: no PV yet; QK^T of tile 1 (steps 0-6, step 7 opens iteration 1) while this
  // tile's weights are formed
  {
    if (v_loader) dma_tile(0, true);
    else if (2 < n_tiles) dma_tile(2, false);
    mask_tile(0, sA);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sB[kb] = f32x16{};
#pragma unroll
    for (int st = 0; st < 7; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sB[kb] = mfma32(rd_k(1, st, kb), qf[st], sB[kb]);
    if (need_ref) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sB[kb] = mfma32(one_op, qm, sB[kb]);
    }
    // stale keys if n_tiles == 1: discarded
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ring[i] = rd_k(1, 7, i);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int kb = k >> 3, r = 2 * (k & 7);
      const uint32_t w = pack_bf16(__builtin_amdgcn_exp2f(sA[kb][r]), __builtin_amdgcn_exp2f(sA[kb][r + 1]));
      pB[k >> 2][k & 3] = w;
      part[k & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, part[k & 3],
                                                    false);
    }
    float rs = (part[0] + part[1]) + (part[2] + part[3]);
    if (__builtin_amdgcn_ballot_w64(!m_valid || !(rs <= 0x1p64f))) slow_path(sA, sB, pB, rs);
    l_run += rs;
    vm_wait();
    __syncthreads();
  }
  // iterations 1.. : S and weights alternate between the A/B register sets
  int j = 1;
  for (; j + 1 < n_tiles; j += 2) {
    iter(j, std::integral_constant<int, 1>{}, sB, sA, pB, pA);
    iter(j + 1, std::integral_constant<int, 0>{}, sA, sB, pA, pB);
  }
  if (j < n_tiles) {
    iter(j, std::integral_constant<int, 1>{}, sB, sA, pB, pA);
    ++j;
  }
  // every wave has passed the last iteration's barrier, so no K buffer is read any more: the next
  // item's first K tiles go out now
  const bool next_k = p.persist && has_next;
  if (next_k && !v_loader) {
    int qt_n, b_n, kvh_n;
    item_coords(vb_next, qt_n, b_n, kvh_n);
    const __amdgpu_buffer_rsrc_t rs_n = kv_rsrc(b_n, kvh_n);
    const int kb_n = item_k_begin(qt_n * MQ);
    // lane offsets recomputed here rather than kept in registers through the tile loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint32_t lds_b = lds_k + 16 * wg * kRow;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t == 0 || item_n_tiles(qt_n * MQ) > 1) {
        const uint32_t row0 = (uint32_t)(kb_n + t * kNk + 16 * wg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * i + (ln >> 4);
          const uint32_t voff = (uint32_t)((ln >> 4) * row_bytes + 16 * ((ln & 15) ^ swz(row)));
          lds_dma16(lds_b + t * kTileBytes + 4 * i * kRow, voff, rs_n, (row0 + 4 * i) * (uint32_t)row_bytes);
        }
      }
    }
  }
  // PV of the last tile (its weights are in the set written last)
  {
    u32x4 (&pl)[4] = ((n_tiles & 1) ? pB : pA);
    const int par = (n_tiles - 1) & 1;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = mfma32(rd_v(par, st, db), __builtin_bit_cast(bf16x8, pl[st]), o[db]);
  }

  // ---- epilogue: normalise, gate, round, store. The MFMA output gives lane (query, hi) dims
  // 4 hi .. 4 hi + 3 of every 8-dim chunk; one v_permlane32_swap per dword hands each lane whole
  // chunks (chunk 2m + hi of the pair 2m, 2m + 1), so every store moves 16 bytes per lane.
  {
    const bool store = my_row < T;
    const float l_tot = l_run + shfl_xor_f(l_run, 32);
    const float inv = 1.0f / l_tot;
    if (p.lse && hi == 0 && store)  // scores are in log2 units relative to m_ref
      p.lse[((int64_t)b * T + my_row) * p.Hq + head] = (m_ref + __log2f(l_tot)) * 0.6931471805599453f;
    const int64_t tok = (int64_t)b * T + min(my_row, T - 1);
    uint16_t* dst = p.out + tok * p.so + (int64_t)head * kHeadDim;
    const uint16_t* gsrc = GATED ? p.gate + tok * p.sg + (int64_t)head * kHeadDim : nullptr;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t w[4];  // output-layout words of chunks 2m (w[0..1]) and 2m + 1 (w[2..3])
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int cidx = 2 * m + hh, db = cidx >> 2, rq = cidx & 3;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = o[db][4 * rq + j] * inv;
        if (GATED) {
          const u32x2 g = *reinterpret_cast<const u32x2*>(gsrc + 32 * db + 8 * rq + 4 * hi);
          const float gv[4] = {bf16lo(g[0]), bf16hi(g[0]), bf16lo(g[1]), bf16hi(g[1])};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            y[j] *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv[j] * 1.4426950408889634f));
        }
        w[2 * hh] = pack_bf16(y[0], y[1]);
        w[2 * hh + 1] = pack_bf16(y[2], y[3]);
      }
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const auto sw = __builtin_amdgcn_permlane32_swap(w[d], w[d + 2], false, false);
        w[d] = sw[0];
        w[d + 2] = sw[1];
      }
      if (store) *reinterpret_cast<u32x4*>(dst + 8 * (2 * m + hi)) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
  q_ready = prefetch_q;
  k_ready = next_k;
  vb = vb_next;
  ++item_k;
  }  // items
}

// ---------------------------------------------------------------------------------------------
// Cache hand-off: copies of whole token rows between caches and staging buffers, 16 bytes per
// lane (the pages' KV-cache layout: local layers a ring of the last window positions, global
// layers one row per position; zh-TW translation page, section 2.3).
__device__ __forceinline__ void copy_rows(const RowCopyParams& p) {
  const int lanes_per_row = p.row_elems / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_seq = (int64_t)p.rows * lanes_per_row;
  if (i >= per_seq * p.B) return;
  const int64_t b = i / per_seq;
  const int64_t rem = i - b * per_seq;
  const int64_t j = rem / lanes_per_row;
  const int c = (int)(rem - j * lanes_per_row);
  int64_t rs = p.src_row0 + j, rd = p.dst_row0 + j;
  if (p.src_ring > 0) rs %= p.src_ring;
  if (p.dst_ring > 0) rd %= p.dst_ring;
  u32x4 v = *reinterpret_cast<const u32x4*>(p.src + (b * p.src_bstride + rs) * p.src_stride + 8 * c);
  if (p.fold) {
    float x[8];
    unpack8(v, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = (8 * c + e) & (kHeadDim - 1);
      x[e] *= (d >= p.rot_dim && p.fold_w) ? p.fold_scale * p.fold_w[d] : p.fold_scale;
    }
    v = pack8(x);
  }
  *reinterpret_cast<u32x4*>(p.dst + (b * p.dst_bstride + rd) * p.dst_stride + 8 * c) = v;
}

// Up to three independent copies in one launch: blockIdx.y picks the copy.
struct RowCopyBatch {
  RowCopyParams job[3];
};

__global__ __launch_bounds__(256) void row_copy_kernel(RowCopyBatch pb) {
  switch (blockIdx.y) {
    case 0: copy_rows(pb.job[0]); break;
    case 1: copy_rows(pb.job[1]); break;
    default: copy_rows(pb.job[2]); break;
  }
}

hipError_t launch_row_copies(const RowCopyParams* jobs, int n, hipStream_t s) {
  if (n < 1 || n > 3) return hipErrorInvalidValue;
  RowCopyBatch pb{};
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    pb.job[i] = jobs[i];
    const int64_t e = (int64_t)jobs[i].B * jobs[i].rows * (jobs[i].row_elems / 8);
    blocks = std::max<int64_t>(blocks, (e + 255) / 256);
  }
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(row_copy_kernel, dim3((unsigned)blocks, (unsigned)n), dim3(256), 0, s, pb);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_kprep(const KPrepParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.T * p.Hkv;
  if (rows == 0) return hipSuccess;
  // 32 rows per block per pass; at most 8 blocks per CU (256 CUs), the waves stride over the rest
  const int64_t blocks = std::min<int64_t>((rows + 31) / 32, 256 * 8);
  hipLaunchKernelGGL(kprep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int G, bool GATED>
static hipError_t launch_prefill_t(const PrefillParams& p_in, hipStream_t s) {
  constexpr int lds = kLdsBytes;
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = prefill_kernel<G, GATED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  PrefillParams p = p_in;
  int64_t grid = (int64_t)p.n_qtiles * p.B * p.Hkv;
  // Full causal layers with many items run persistent: one workgroup per CU (the LDS allows one),
  // the CUs of an XCD sharing its (sequence, KV head) pairs as the item order expects. The q rows
  // prefetched for the next item are read through one buffer resource per sequence, whose byte
  // range must stay below 2^32.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      p.window == 0 && p.rope.half == 21 && (p.B * p.Hkv) % 8 == 0 && cus > 0 && cus % 8 == 0 &&
      grid >= 2 * (int64_t)cus && (int64_t)p.T * p.sq * 2 < (int64_t)1 << 32) {
    p.persist = 1;
    grid = cus;
  } else {
    p.persist = 0;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int group, bool gated, hipStream_t s) {
  if (p.qoff == 0 && p.kv_rows == p.T && prefill_uses_swa(p.window, group, p.rope.half))
    return launch_prefill_swa(p, gated, s);
  return launch_prefill_general(p, group, gated, s);
}

hipError_t launch_prefill_general(const PrefillParams& p, int group, bool gated, hipStream_t s) {
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
