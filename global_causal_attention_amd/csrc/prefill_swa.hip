// Prefill attention for banded layers with a window of at most 128 keys, four query heads per KV
// head and 42 rotary dims: a streaming kernel in which each workgroup walks a run of 64-query steps
// of one (sequence, KV head). The general tiled kernel (prefill.hip) covers every other shape.
//
// Method: ZGCM-1 zh-TW translation page, section 2.1 "Model overview" and Figure 3 (GQA 32/8 heads
// of dim 128, 128-token window on local layers, QK-RMSNorm, partial RoPE over a third of the head,
// output multiplied by the sigmoid of a gate projection).
#include <cstddef>
#include <type_traits>

#include "zg_mfma.hpp"

namespace zg {

namespace {

// ---------------------------------------------------------------------------------------------
// Streaming kernel for banded layers with window <= 128, four query heads per KV head and a
// rotary dimension of 42 (21 pairs).
//
// A workgroup walks a run of 64-query steps of one (sequence b, KV head); wave w owns query head
// w % 4 and 32 queries (block w / 4) of each step. A step needs its own 64 keys and the 128 before
// them, i.e. three 64-key tiles, so K and V tiles sit in a three-slot LDS ring and each step brings
// in exactly one new tile, issued at the top of the step into the slot of a tile the previous
// step read only before its mid-step barrier; the new tile's key blocks are visited last, behind
// the q prologue and the blocks of the two older tiles, and one barrier per step (before those
// blocks) is the only synchronisation. Each wave's raw q rows for the next step stream into its own 8 KB LDS area as soon as the
// prologue has turned this step's rows into MFMA operands; the gate rows come into registers during
// the step. Loads are tracked with explicit vmcnt waits, so no wait covers a load issued for a
// later phase.
//
// Arithmetic layout. The score of query i and key j in log2 units is
//   inv_i * (q'_i . k''_j),  inv_i = 1 / sqrt(mean(q_i^2) + eps),
// where q'_i is the raw q row with its first 42 dims replaced by RoPE(w_q * q_i) (rounded to bf16)
// and k''_j is the prepared key with the softmax scale * log2(e), and for dims >= 42 the q norm
// weight, folded in (the keys are prepared with KPrepParams::fold). The RMS factor is applied to
// the scores instead of the q rows, so 86 of the 128 q dims reach the matrix cores as loaded.
//
// Tile layout in LDS (K and V alike): 64 rows in 16 groups of 4 rows; group g occupies 1 KB as
// [16-byte chunk][row of the group], with chunk c stored at position c ^ (g & 3). Each
// buffer_load ... lds fills one group (4 whole rows, so global reads stay row-contiguous), the
// 16-row QK^T operand reads and the 4-row transposing PV reads both hit 64 distinct banks, and every
// operand address is a per-lane base plus an immediate.
constexpr int kSwaRotHalf = 21;
constexpr int kSwaTile = 16 * 1024;
constexpr int kSwaSlot = 2 * kSwaTile;      // K tile, then V tile
constexpr int kSwaRing = 3 * kSwaSlot;
constexpr int kSwaQArea = 32 * 256;         // per wave: 32 q rows
constexpr int kSwaLds = kSwaRing + kWaves * kSwaQArea;
static_assert(kSwaLds <= 160 * 1024, "LDS budget");

}  // namespace

template <bool GATED>
__global__ __launch_bounds__(kThreads) void prefill_swa_kernel(PrefillParams p) {
  constexpr int HR = kSwaRotHalf;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int per_seg = p.B * p.Hkv;
  const int seg = blockIdx.x / per_seg;
  const int bh = blockIdx.x - seg * per_seg;
  const int b = bh / p.Hkv;
  const int kvh = bh - b * p.Hkv;
  const int T = p.T;
  const int W = p.window;
  const int hg = wave & 3;
  const int qb = wave >> 2;
  const int head = kvh * 4 + hg;
  const int t_seg0 = seg * p.seg_steps;   // first 64-query step of the run
  const int n_steps = min(p.seg_steps, (T + 63) / 64 - t_seg0);
  // Query row t reads key rows up to qoff + t (qoff > 0: a cached context precedes the new
  // rows). The newest key tile of step tc is tq0 + tc; with qoff = 0 or 63 (mod 64) and W <= 128
  // a step's keys span at most three 64-key tiles, which the ring holds.
  const int qoff = p.qoff;
  const int tq0 = (qoff + 63) >> 6;

  // ---- K/V tiles: waves 0-3 bring K row groups 4 wg .. 4 wg + 3, waves 4-7 the V ones
  const bool v_loader = wave >= 4;
  const int wg = wave & 3;
  const int row_bytes = (int)((v_loader ? p.sv : (int64_t)p.Hkv * kHeadDim) * 2);
  const uint16_t* slab = v_loader ? p.v + (int64_t)b * p.kv_rows * p.sv + (int64_t)kvh * kHeadDim
                                  : p.khat + ((int64_t)b * p.kv_rows * p.Hkv + kvh) * kHeadDim;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)slab, 0, (int)((uint32_t)p.n_keys * (uint32_t)row_bytes),
                                        0x00020000);  // byte count < 2^32, read as unsigned
  const uint32_t lds_kv = (uint32_t)(uintptr_t)smem + (v_loader ? kSwaTile : 0);
  auto dma_tile = [&](int t) {  // tile t (rows 64t .. 64t + 63) into ring slot t % 3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * wg + i;  // g & 3 == i
      const uint32_t m0v = lds_kv + (t % 3) * kSwaSlot + g * 1024;
      const uint32_t soff = (uint32_t)(64 * t + 4 * g) * (uint32_t)row_bytes;
      const uint32_t voff = (uint32_t)((lane & 3) * row_bytes + 16 * ((lane >> 2) ^ i));
      lds_dma16(m0v, voff, rsrc, soff);
    }
  };

  // ---- raw q rows of this wave: row r at r * 256, chunk c at position c ^ (r & 15)
  const int q_row_bytes = (int)(p.sq * 2);
  const __amdgpu_buffer_rsrc_t rsrc_q = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.q + (int64_t)b * T * p.sq + (int64_t)head * kHeadDim), 0,
      (int)((uint32_t)T * (uint32_t)q_row_bytes),
      0x00020000);
  unsigned char* qs = smem + kSwaRing + wave * kSwaQArea;
  const uint32_t lds_q = (uint32_t)(uintptr_t)qs;
  auto dma_q = [&](int step) {  // 32 rows, 4 per instruction
    const int row0 = 64 * (t_seg0 + step) + 32 * qb;
    // the area's previous contents (this step's operands) must have been read out first
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      const uint32_t m0v = lds_q + i * 1024;
      const uint32_t soff = (uint32_t)(row0 + 4 * i) * (uint32_t)q_row_bytes;
      const uint32_t voff = (uint32_t)((lane >> 4) * q_row_bytes + 16 * ((lane & 15) ^ (r & 15)));
      lds_dma16(m0v, voff, rsrc_q, soff);
    }
  };
  // B-operand read of step st: chunk 2 st + hi of row l32, i.e. q_op0 + 32 (st ^ q_opx)
  const int q_op0 = l32 * 256 + 16 * (hi ^ (l32 & 1));
  const int q_opx = (l32 >> 1) & 7;

  // ---- per-lane operand offsets
  // QK^T A operand (key row l32 of a 32-key block, chunk 2 st + hi): even and odd st differ in
  // how the group swizzle moves the chunk
  const int kx = (l32 >> 2) & 3;
  const int k_lane = (l32 >> 2) * 1024 + (l32 & 3) * 16 + 64 * (hi ^ (kx & 1));
  const int k_even = k_lane + 128 * (kx >> 1);
  const int k_odd = k_lane - 128 * (kx >> 1);
  // PV A operand: transposing read x of key step st covers row group 4 st + 2 x + hi
  int v_lane[2];
  {
    const int u = (lane & 15) >> 2;
    const int dch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int gx = 2 * x + hi;
      v_lane[x] = kSwaTile + gx * 1024 + (dch ^ gx) * 64 + u * 16 + 8 * (lane & 1);
    }
  }
  const bf16x8 one_op = hi ? bf16x8{} : bf16x8{(__bf16)1.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f,
                                               (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int key_lane = 4 * hi;  // key offset of this lane's score registers within a block

  // Gate rows and output rows move as whole 16-byte chunks: lane (row q, hi) holds chunks
  // 2 m + hi (m = 0..7) of row q. The MFMA output layout gives each lane 4-dim halves of every
  // chunk instead; one v_permlane32_swap per dword converts between the two (chunk pair 2m, 2m+1).
  u32x4 gch[8];
  auto load_gate = [&](int step) {
    const int t = 64 * (t_seg0 + step) + 32 * qb + l32;
    const uint16_t* g = p.gate + ((int64_t)b * T + min(t, T - 1)) * p.sg + (int64_t)head * kHeadDim;
#pragma unroll
    for (int m = 0; m < 8; ++m) gch[m] = *reinterpret_cast<const u32x4*>(g + 8 * (2 * m + hi));
  };

  // ---- start of the run: the tiles before the first step's newest one, and the first q rows
  {
    const int t_first = max(0, (qoff + 64 * t_seg0 - W + 1) >> 6);
    for (int t = t_first; t < tq0 + t_seg0; ++t) dma_tile(t);
    dma_q(0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }

  for (int step = 0; step < n_steps; ++step) {
    const int tc = t_seg0 + step;           // this step's query rows 64 tc .. 64 tc + 63
    const int qbase = 64 * tc + 32 * qb;
    const int my_q = qbase + l32;
    const int qk = qoff + qbase;            // key row of this wave's first query
    const bool has_next = step + 1 < n_steps;
    dma_tile(tq0 + tc);

    // -- q prologue (raw rows landed before the previous epilogue). Lane pair (r, half) holds dims
    // 64 half .. 64 half + 63 of row r: sum of squares for the RMS factor, and on half 0 the
    // rotation of dims 0..41 (weighted), written back in place as bf16.
    float inv_q;
    {
      const int r = lane >> 1;
      const int half = lane & 1;
      u32x4 raw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        raw[i] = *reinterpret_cast<const u32x4*>(qs + r * 256 + 16 * ((8 * half + i) ^ (r & 15)));
      float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          // (the words go through scalars: a bit_cast of a vector element reads element 0 with
          // this compiler)
          const uint32_t w0 = raw[i][j], w1 = raw[i][j + 1];
          const bf16x2 a0 = __builtin_bit_cast(bf16x2, w0), a1 = __builtin_bit_cast(bf16x2, w1);
          ss0 = __builtin_amdgcn_fdot2_f32_bf16(a0, a0, ss0, false);
          ss1 = __builtin_amdgcn_fdot2_f32_bf16(a1, a1, ss1, false);
        }
      float ss = ss0 + ss1;
      ss += dpp_swap_pair(ss);
      const float inv_row = rsqrtf(ss * (1.0f / kHeadDim) + p.eps);
      // rotary angles: half 0 computes pairs 0..10, half 1 pairs 11..20; half 0 takes the second
      // set from its partner lane
      typedef __attribute__((address_space(4))) const unsigned char* karg_ptr;
      karg_ptr ka = (karg_ptr)__builtin_amdgcn_kernarg_segment_ptr();
      asm volatile("" : "+s"(ka));
      const RopeTable& rt = *(const RopeTable*)(ka + offsetof(PrefillParams, rope));
      const int64_t pos = p.pos0 + qbase + r;
      float cs[HR], sn[HR];
#pragma unroll
      for (int j = 0; j < 11; ++j) {
        double rev0 = rt.rev[j], rev1 = rt.rev[min(j + 11, HR - 1)];
        asm("" : "+s"(rev0), "+s"(rev1));  // scalar loads; the lane picks its pair
        const double rev = half ? rev1 : rev0;
        float c_, s_;
        rope_cs(pos, rev, c_, s_);
        if (j < 11) { cs[j] = c_; sn[j] = s_; }
        if (j + 11 < HR) {
          cs[j + 11] = dpp_swap_pair(c_);
          sn[j + 11] = dpp_swap_pair(s_);
        }
      }
      if (half == 0) {
        const_f32_ptr w = (const_f32_ptr)p.q_norm_w;
        float x[2 * HR];
#pragma unroll
        for (int d = 0; d < 2 * HR; ++d) {
          const uint32_t word = raw[d >> 3][(d & 7) >> 1];
          x[d] = (d & 1) ? bf16hi(word) : bf16lo(word);
          if (w) {
            float wd = w[d];
            asm("" : "+s"(wd));
            x[d] *= wd;
          }
        }
#pragma unroll
        for (int i = 0; i < HR; ++i) {
          const float a = x[i], bb = x[i + HR];
          x[i] = a * cs[i] - bb * sn[i];
          x[i + HR] = bb * cs[i] + a * sn[i];
        }
#pragma unroll
        for (int d = 0; d < 2 * HR; d += 2) raw[d >> 3][(d & 7) >> 1] = pack_bf16(x[d], x[d + 1]);
#pragma unroll
        for (int i = 0; i < 6; ++i)
          *reinterpret_cast<u32x4*>(qs + r * 256 + 16 * (i ^ (r & 15))) = raw[i];
      }
      inv_q = __shfl(inv_row, 2 * l32, 64);
    }
    bf16x8 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qs + q_op0 + 32 * (s ^ q_opx));
    if (has_next) dma_q(step + 1);
    if (GATED) load_gate(step);

    // -- attention over the 32-key blocks [kb_lo, kb_hi]: the blocks of older tiles newest first,
    // then those of tile tc. Softmax weights are exp2(inv_q * (s - mu)) with a bf16 reference mu
    // per query (subtracted by a ninth MFMA step), raised only when a partial sum leaves
    // [0, 2^64] or no key has been seen yet; the first block of a step sets it from its maximum.
    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x16{};
    float l_run = 0.f;
    float mu = 0.f;
    bool m_valid = false;
    bf16x8 qm = bf16x8{};
    auto block = [&](int kb, auto first_c) {
      constexpr bool first = decltype(first_c)::value;
      const int slot = ((kb >> 1) % 3) * kSwaSlot + (kb & 1) * 8192;
      const unsigned char* kp = smem + slot;
      f32x16 s = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st)
        s = mfma32(*reinterpret_cast<const bf16x8*>(kp + ((st & 1) ? k_odd : k_even) + 128 * st), qf[st], s);
      if constexpr (!first) s = mfma32(one_op, qm, s);
      // masks: key k0 + c_r + 4 hi is valid for the query at key row qoff + my_q when
      // 0 <= qoff + my_q - key < W, i.e. when (unsigned)(t - c_r) < W with t = qoff + my_q - k0 - 4 hi
      const int k0 = 32 * kb;
      if (k0 + 31 > qk || k0 < qk + 32 - W) {
        const uint32_t t = (uint32_t)(qoff + my_q - k0 - key_lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t cr = 8 * (r >> 2) + (r & 3);
          s[r] = (t - cr < (uint32_t)W) ? s[r] : -INFINITY;
        }
      }
      u32x4 pk[2];
      float rs;
      if constexpr (first) {
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(mx, __uint_as_float(hi ? sw[0] : sw[1]));
        m_valid = mx > -INFINITY;
        mu = m_valid ? bf16lo(pack_bf16(mx, 0.f)) : 0.f;
        const float nmu = -inv_q * mu;
        float pt = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t w = pack_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(inv_q, s[2 * k], nmu)),
                                       __builtin_amdgcn_exp2f(__builtin_fmaf(inv_q, s[2 * k + 1], nmu)));
          pk[k >> 2][k & 3] = w;
          pt = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, pt, false);
        }
        rs = pt;
        qm = hi ? bf16x8{} : bf16x8{(__bf16)(-mu), (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f,
                                    (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
      } else {
        float part[2] = {0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t w = pack_bf16(__builtin_amdgcn_exp2f(inv_q * s[2 * k]),
                                       __builtin_amdgcn_exp2f(inv_q * s[2 * k + 1]));
          pk[k >> 2][k & 3] = w;
          part[k & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, part[k & 1], false);
        }
        rs = part[0] + part[1];
        if (__builtin_amdgcn_ballot_w64(!m_valid || !(rs <= 0x1p64f))) {
          float mx = s[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(mx, __uint_as_float(hi ? sw[0] : sw[1])) + mu;
          const bool has = mx > -INFINITY;
          float mu_new = m_valid ? fmaxf(mu, mx) : mx;
          mu_new = has || m_valid ? bf16lo(pack_bf16(mu_new, 0.f)) : mu;
          const float delta = mu - mu_new;
          const float alpha = m_valid ? __builtin_amdgcn_exp2f(inv_q * delta) : 0.f;
          l_run *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] *= alpha;
          float pt = 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t w = pack_bf16(__builtin_amdgcn_exp2f(inv_q * (s[2 * k] + delta)),
                                         __builtin_amdgcn_exp2f(inv_q * (s[2 * k + 1] + delta)));
            pk[k >> 2][k & 3] = w;
            pt = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, pt, false);
          }
          rs = pt;
          mu = mu_new;
          m_valid = m_valid || has;
          qm = hi ? bf16x8{} : bf16x8{(__bf16)(-mu), (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f,
                                      (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
        }
      }
      l_run += rs;
      const unsigned char* vp = smem + slot;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const i16x4 lo4 = lds_read_tr(vp + v_lane[0] + 4096 * st + 256 * db);
          const i16x4 hi4 = lds_read_tr(vp + v_lane[1] + 4096 * st + 256 * db);
          const i16x4 both[2] = {lo4, hi4};
          o[db] = mfma32(__builtin_bit_cast(bf16x8, both), __builtin_bit_cast(bf16x8, pk[st]), o[db]);
        }
    };
    const int kb_lo = max(0, (qk - W + 1) >> 5);
    const int kb_hi = (qk + 31) >> 5;
    const int kb_new = 2 * (tq0 + tc);  // first block of the newest tile (kb_hi >= kb_new)
    // tile tc has landed once every wave's share of it has; only the loads issued after it (next
    // q rows: 8 instructions, gate: 8) may still be in flight
    auto wait_new_tile = [&]() {
      if (GATED) {
        if (has_next) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
      } else {
        if (has_next) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      }
    };
    using First = std::integral_constant<bool, true>;
    using Rest = std::integral_constant<bool, false>;
    const int kb_old = min(kb_hi, kb_new - 1);  // newest block of an older tile
    int kb2 = max(kb_lo, kb_new);
    if (kb_old >= kb_lo) {
      block(kb_old, First{});
      for (int kb = kb_old - 1; kb >= kb_lo; --kb) block(kb, Rest{});
      wait_new_tile();
    } else {
      wait_new_tile();
      block(kb2++, First{});
    }
    for (int kb = kb2; kb <= kb_hi; ++kb) block(kb, Rest{});

    // -- epilogue: every load of this step (gate, next q rows) has landed past this wait, which is
    // issued through the builtin so that the compiler's own wait tracking knows it too (the gate
    // registers are then free for the next prologue without further waits)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt: no wait
    {
      const float l_tot = l_run + shfl_xor_f(l_run, 32);
      // (a gate of 0 then gives exactly half the ungated output: rcp(2 l) = rcp(l) / 2)
      const float rcp_l = __builtin_amdgcn_rcpf(l_tot);
      const bool store = my_q < T;
      // the row's natural-log log-sum-exp for the backward pass: the weights are exp2 of
      // inv_q * (s - mu), so log2 of the row's sum of exp2(inv_q * s) is inv_q * mu + log2(l)
      if (p.lse && hi == 0 && store)
        p.lse[((int64_t)b * T + my_q) * p.Hq + head] =
            (inv_q * mu + __log2f(l_tot)) * 0.6931471805599453f;
      uint16_t* dst = p.out + ((int64_t)b * T + min(my_q, T - 1)) * p.so + (int64_t)head * kHeadDim;
      if (GATED) {
        // chunks -> output layout: dims 8c + 4 hi .. + 3 of chunk c in half (c & 1) of gch[c / 2]
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const auto sw = __builtin_amdgcn_permlane32_swap(gch[m][d], gch[m][d + 2], false, false);
            gch[m][d] = sw[0];
            gch[m][d + 2] = sw[1];
          }
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t w[4];  // output layout words of chunks 2m (w[0..1]) and 2m + 1 (w[2..3])
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = 2 * m + h, db = c >> 2, rq = c & 3;
          float y[4];
          if (GATED) {
            // o / (l * (1 + exp(-g))): one reciprocal per element covers both divisions
            const uint32_t g0 = gch[m][2 * h], g1 = gch[m][2 * h + 1];
            const float gv[4] = {bf16lo(g0), bf16hi(g0), bf16lo(g1), bf16hi(g1)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float e = __builtin_amdgcn_exp2f(-gv[j] * 1.4426950408889634f);
              y[j] = o[db][4 * rq + j] * __builtin_amdgcn_rcpf(__builtin_fmaf(l_tot, e, l_tot));
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = o[db][4 * rq + j] * rcp_l;
          }
          w[2 * h] = pack_bf16(y[0], y[1]);
          w[2 * h + 1] = pack_bf16(y[2], y[3]);
        }
        // output layout -> chunk 2m + hi of this lane's row
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto sw = __builtin_amdgcn_permlane32_swap(w[d], w[d + 2], false, false);
          w[d] = sw[0];
          w[d + 2] = sw[1];
        }
        if (store)
          *reinterpret_cast<u32x4*>(dst + 8 * (2 * m + hi)) = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
    // No barrier here: the slot the next step refills held a tile that only the older-tile blocks
    // of this step read, and every wave finished those before the barrier above.
  }
}

template <bool GATED>
static hipError_t launch_swa_t(const PrefillParams& p, hipStream_t s) {
  auto kern = prefill_swa_kernel<GATED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kSwaLds);
  if (e != hipSuccess) return e;
  if (p.seg_steps < 1) return hipErrorInvalidValue;
  const int64_t n_seg = ((int64_t)p.T + 64 * p.seg_steps - 1) / (64 * p.seg_steps);
  const int64_t grid = n_seg * p.B * p.Hkv;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), kSwaLds, s, p);
  return hipGetLastError();
}

bool prefill_uses_swa(int window, int group, int rot_half) {
  return window > 0 && window <= 128 && group == 4 && rot_half == kSwaRotHalf;
}

bool prefill_swa_offset_ok(int64_t qoff, int window) {
  // a step's key rows [qoff + 64 tc - W + 1, qoff + 64 tc + 63] must span at most three 64-key
  // tiles, and every wave's queries must reach the step's newest tile (qoff = 0 or 63 mod 64)
  const int64_t r = qoff & 63;
  return window > 0 && window <= 128 && (r == 0 || r == 63) &&
         ((qoff - window + 1) & 63) <= 129 - window;
}

hipError_t launch_prefill_swa(const PrefillParams& p, bool gated, hipStream_t s) {
  return gated ? launch_swa_t<true>(p, s) : launch_swa_t<false>(p, s);
}

}  // namespace zg
