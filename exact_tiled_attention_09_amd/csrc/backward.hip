// Attention backward for gfx950: gradients dQ, dK, dV of O = softmax(scale Q K^T) V, bf16 in / bf16 out,
// fp32 accumulation.
//
// The probabilities are recomputed from Q, K and the forward's log-sum-exp instead of being stored
// ("How FlashAttention Speeds Up LLM Attention", table of contents: recompute probabilities for
// training; "FlashAttention Explained: How AI Models Process Attention Faster and Use Less Memory",
// "FlashAttention in AI Training", "More Efficient Backpropagation").  With the LSE known, a tile's
// probabilities are final at once: P = 2^(s*c - LSE*log2 e), c = scale*log2 e.  The gradients are the
// plain derivative of the attention function:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = rowsum(dO_i * O_i) = rowsum(P_i * dP_i),
//   dQ = scale dS K,  dK = scale dS^T Q.
// Two kernels, no atomics (every output element is summed by one lane, in a fixed order):
//  * bwd_dq_kernel: one work-group per (b, h, 128 queries); the layout of the forward kernel (S^T = K Q^T
//    with a lane pair per query).  It also computes D from dO and O and stores it for the next kernel.
//    Per 64-key tile: S^T = K Q^T and dP^T = V dO^T (K, V fragments from LDS), dS^T in registers,
//    dQ^T += K^T dS^T (K^T through ds_read_b64_tr_b16 of the same K tile).
//  * bwd_dkdv_kernel: one work-group per (b, h, 256 keys at d = 128, 128 at d = 64), the same layout
//    with the roles of queries and keys exchanged (S = Q K^T with a lane pair per key).  Per 32-query
//    block of the 64-query tiles streamed through LDS: S = Q K^T, dP = dO V^T, then dV^T += dO^T P and
//    dK^T += Q^T dS (dO^T, Q^T through transposing reads), both gradients in one pass.
// Tiles read both row-wise (ds_read_b128) and transposed (ds_read_b64_tr_b16) use a swizzle that keeps
// both access patterns on distinct banks.
#include "common.h"
#include "kernels.h"
#include "lds_tiles.h"

namespace fa {

struct BwdParams {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  const uint16_t* __restrict__ o;
  const uint16_t* __restrict__ dout;
  const float* __restrict__ lse;
  float* __restrict__ delta;  // D [B,H,N_q], written by bwd_dq_kernel, read by bwd_dkdv_kernel
  uint16_t* __restrict__ dq;
  uint16_t* __restrict__ dk;
  uint16_t* __restrict__ dv;
  int Nq, Nkv, off;
  int n_qt, n_kt;            // 128-query blocks (dQ kernel) and key blocks of the dK/dV kernel per (b, h)
  int total_q, total_k;      // work-groups of the two kernels
  int pair_q, pair_k;        // causal: one work-group runs blocks j and n-1-j (equal work per group)
  float c;                   // scale * log2(e) (any sign)
  float scale;
};

template <int D>
struct BwdCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int BR = 128;           // queries (dQ kernel) or keys (dK/dV kernel) per work-group
  static constexpr int BC = 64;            // keys per tile in the dQ kernel
  static constexpr int ROWB = 2 * D, CH = D / 8, KS = D / 16, MBD = D / 32, RPL = 1024 / ROWB;
  static constexpr int NBLK = BC / 32;
  static constexpr int TKV = BC * ROWB;
  static constexpr int LPT_KV = TKV / (NT * 16);
  static_assert(TKV % (NT * 16) == 0 && 32 * ROWB % (NT * 16) == 0, "tile loads must divide evenly");
};

// Row swizzle (16-byte chunk XOR) for tiles that are read both as MFMA rows and through
// ds_read_b64_tr_b16.  The LDS serves 64 banks of 4 bytes (256 bytes) per cycle: a ds_read_b128 in
// passes of 16 lanes, a ds_read_b64_tr_b16 in passes of 32.  Row reads put 16 rows at one logical chunk
// into a pass, so the XOR must be a bijection over those rows; transposing reads put 4 consecutive rows
// times 4 consecutive chunks (one aligned group of 4) into a pass, so the 4 rows must XOR their chunks
// into distinct groups of 4.  d = 128 (a row is exactly the 64 banks): bits 2-3 of the XOR come from
// r % 4, bits 0-1 from r / 4 % 4.  d = 64 (two rows per 256 bytes): rows of equal parity share a bank
// half; bit 2 from r / 2 % 2, bits 0-1 from r / 4 % 4.
template <int D>
__device__ __forceinline__ int swz_kv(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Per-lane LDS byte offsets of the two transposing reads (u = 0, 1: rows 8u + 4h + j/4 of a 16-row
// chunk) for the d block mbd: lane i of each 16-lane group then holds element [row0 + t][32 mbd + 16 dh
// + i], t = 0..3, the A-operand layout of a 32-row (d) by 16-column (rows of the tile) MFMA fragment.
template <int D>
__device__ __forceinline__ int tr_offset(int lane, int mbd, int u) {
  using C = BwdCfg<D>;
  const int h = lane >> 5, j = lane & 15, dh = (lane >> 4) & 1;
  const int row = 8 * u + 4 * h + j / 4;
  const int d0 = 32 * mbd + 16 * dh + 4 * (j & 3);
  return row * C::ROWB + 16 * ((d0 >> 3) ^ swz_kv<D>(row)) + 2 * (d0 & 7);
}

template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const uint8_t* base, const int (&off)[2]) {
  const s16x4 lo = lds_read_tr16(base + off[0]);
  const s16x4 hi = lds_read_tr16(base + off[1]);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float dot8_f32(u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(bf16lo_to_f32(a[i]), bf16lo_to_f32(b[i]), s);
    s = fmaf(bf16hi_to_f32(a[i]), bf16hi_to_f32(b[i]), s);
  }
  return s;
}

// Stores a 32 (d) x 32 (rows) fp32 MFMA accumulator block, times `mul`, as bf16 into row `row` (this
// lane's column) of a row-major [., D] tensor: elements 8g + 4h + 0..3 of the block are contiguous in d.
template <int D>
__device__ __forceinline__ void store_rowT(uint16_t* rowp, const f32x16 (&acc)[D / 32], float mul, int h) {
#pragma unroll
  for (int mbd = 0; mbd < D / 32; ++mbd)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2 val;
      val[0] = pack_bf16x2(acc[mbd][4 * g4 + 0] * mul, acc[mbd][4 * g4 + 1] * mul);
      val[1] = pack_bf16x2(acc[mbd][4 * g4 + 2] * mul, acc[mbd][4 * g4 + 3] * mul);
      *reinterpret_cast<u32x2*>(rowp + mbd * 32 + 8 * g4 + 4 * h) = val;
    }
}

// ------------------------------------------------------------------------------------------- dQ (and D)

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lk0[C::TKV], lv0[C::TKV], lk1[C::TKV], lv1[C::TKV];
  auto kbuf = [&](int st) -> uint8_t* { return st == 0 ? lk0 : lk1; };
  auto vbuf = [&](int st) -> uint8_t* { return st == 0 ? lv0 : lv1; };

  const int lid = xcd_logical_id(blockIdx.x, p.total_q);
  const bool pair = CAUSAL && p.pair_q;
  const int per_bh = pair ? (p.n_qt + 1) / 2 : p.n_qt;
  const int bh = lid / per_bh;
  const int qt_lo = lid - bh * per_bh;
  const int qt_hi = CAUSAL ? p.n_qt - 1 - qt_lo : qt_lo;  // heaviest query blocks first
  const int n_pass = (pair && qt_lo != qt_hi) ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    const int qt = pass == 0 ? qt_hi : qt_lo;
    if (pass > 0) __syncthreads();  // every wave is done with the LDS stages before they are refilled
    const int q0 = qt * C::BR;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // lane offsets are recomputed per pass, not held across both
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const size_t head_q = (size_t)bh * p.Nq * D, head_kv = (size_t)bh * p.Nkv * D;
    const uint16_t* __restrict__ kg = p.k + head_kv;
    const uint16_t* __restrict__ vg = p.v + head_kv;
    const int qw0 = q0 + 32 * w, qi = qw0 + l32;
    const bool row_ok = qi < p.Nq;

    // Q^T and dO^T fragments of this lane's query (d = 16 ks + 8 h .. +7), D_i = dO_i . O_i, LSE_i log2 e
    bf16x8 qf[C::KS], dof[C::KS];
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = a, o = a;
      if (row_ok) {
        const size_t e = head_q + (size_t)qi * D + ks * 16 + 8 * h;
        a = load16(p.q + e);
        b = load16(p.dout + e);
        o = load16(p.o + e);
      }
      qf[ks] = __builtin_bit_cast(bf16x8, a);
      dof[ks] = __builtin_bit_cast(bf16x8, b);
      dpart += dot8_f32(b, o);
    }
    const float Di = pair_sum(dpart);
    if (row_ok && h == 0) p.delta[(size_t)bh * p.Nq + qi] = Di;
    const float lse2 = row_ok ? p.lse[(size_t)bh * p.Nq + qi] * kLog2e : 0.f;
    const float c = p.c;

    int kv_end = p.Nkv;
    if (CAUSAL) kv_end = min(p.Nkv, q0 + C::BR + p.off);
    const int n_tiles = (kv_end + C::BC - 1) / C::BC;
    const int wave_kv_end = qw0 >= p.Nq ? 0 : (CAUSAL ? min(p.Nkv, qw0 + 32 + p.off) : p.Nkv);
    const int lim = CAUSAL ? min(p.Nkv - 1, qi + p.off) : p.Nkv - 1;

    f32x16 acc[C::MBD];
#pragma unroll
    for (int mbd = 0; mbd < C::MBD; ++mbd) acc[mbd] = f32x16{};

    int ld_off[C::LPT_KV];
#pragma unroll
    for (int i = 0; i < C::LPT_KV; ++i) {
      const int r = C::RPL * (w * C::LPT_KV + i) + lane / C::CH, pc = lane % C::CH;
      ld_off[i] = r * C::ROWB + 16 * (pc ^ swz_kv<D>(r));
    }
    auto load_tile = [&](int t, int stage) {
      const int kv0 = t * C::BC;
      const int bytes = (p.Nkv - kv0) * C::ROWB;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)kv0 * D, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)kv0 * D, bytes);
#pragma unroll
      for (int i = 0; i < C::LPT_KV; ++i) {
        const int blk = 1024 * (w * C::LPT_KV + i);
        load_lds16(rk, ld_off[i], kbuf(stage) + blk);
        load_lds16(rv, ld_off[i], vbuf(stage) + blk);
      }
    };
    int row_off[C::KS];  // row l32 of a 32-row block, logical chunk 2 ks + h
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) row_off[ks] = l32 * C::ROWB + 16 * ((2 * ks + h) ^ swz_kv<D>(l32));
    int trk[C::MBD][2];
#pragma unroll
    for (int mbd = 0; mbd < C::MBD; ++mbd) {
      trk[mbd][0] = tr_offset<D>(lane, mbd, 0);
      trk[mbd][1] = tr_offset<D>(lane, mbd, 1);
    }

    auto compute_tile = [&](const uint8_t* kb, const uint8_t* vb, bool masked, int kv0, auto&& next) {
      f32x16 S[C::NBLK], dP[C::NBLK];
#pragma unroll
      for (int mb = 0; mb < C::NBLK; ++mb) S[mb] = dP[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < C::NBLK; ++mb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + row_off[ks] + mb * 32 * C::ROWB);
          S[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], S[mb], 0, 0, 0);
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vb + row_off[ks] + mb * 32 * C::ROWB);
          dP[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[ks], dP[mb], 0, 0, 0);
        }
      next();
      // dS^T = P^T (dP^T - D), P^T = 2^(s c - LSE log2 e); masked keys get P = 0
      const int rel = lim - kv0 - 4 * h;
      bf16x8 dsf[2 * C::NBLK];
#pragma unroll
      for (int kc = 0; kc < 2 * C::NBLK; ++kc) {
        float ds[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * (kc & 1) + i, mb = kc >> 1;
          float pr = exp2_hw(fmaf(S[mb][r], c, -lse2));
          if (masked && 32 * mb + 8 * (r >> 2) + (r & 3) > rel) pr = 0.f;
          ds[i] = pr * (dP[mb][r] - Di);
        }
        u32x4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(ds[2 * i], ds[2 * i + 1]);
        dsf[kc] = __builtin_bit_cast(bf16x8, pk);
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int kc = 0; kc < 2 * C::NBLK; ++kc)
#pragma unroll
        for (int mbd = 0; mbd < C::MBD; ++mbd)
          acc[mbd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(kb + 16 * kc * C::ROWB, trk[mbd]), dsf[kc],
                                                             acc[mbd], 0, 0, 0);
    };

    auto tile = [&](auto stage_tag, int t) {
      constexpr int STAGE = decltype(stage_tag)::value;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const bool more = t + 1 < n_tiles;
      auto next = [&]() {
        if (more) load_tile(t + 1, STAGE ^ 1);
      };
      const int kv0 = t * C::BC;
      if (kv0 < wave_kv_end)
        compute_tile(kbuf(STAGE), vbuf(STAGE), (kv0 + C::BC > p.Nkv) || (CAUSAL && kv0 + C::BC - 1 > qw0 + p.off),
                     kv0, next);
      else if (more)
        load_tile(t + 1, STAGE ^ 1);
    };

    load_tile(0, 0);
    for (int t = 0; t < n_tiles; t += 2) {
      tile(std::integral_constant<int, 0>{}, t);
      if (t + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, t + 1);
    }
    if (row_ok) store_rowT<D>(p.dq + head_q + (size_t)qi * D, acc, p.scale, h);
  }
}

// ----------------------------------------------------------------------------------------------- dK, dV

// One pass forms both gradients from one S and dP per 32x32 key-query block (D/4 MFMAs; separate dV
// and dK passes would need 5 D/16 and stream Q, dO twice), holding both D x 32 accumulators and the
// wave's K fragments in registers and the work-group's V rows in LDS.  At d = 128 the work-group has 8
// waves (256 keys): the V rows (64 KB) and the Q / dO stages (64 KB) fit one work-group per CU, which
// still runs two waves per SIMD, and each streamed Q / dO tile serves twice as many keys.  (With 4 waves
// and V in registers instead, to keep two work-groups per CU, the compiler spilled 24-45 VGPRs and the
// backward ran 11-13% slower.)  At d = 64, 4 waves and 49 KB of LDS run three waves per SIMD.
template <int D>
struct DkdvShape {  // work-group shape of bwd_dkdv_kernel: waves (32 keys each), threads, groups per CU
  static constexpr int NW = D == 128 ? 8 : 4, NT = 64 * NW, BR = 32 * NW, OCC = D == 128 ? 1 : 2;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DkdvShape<D>::NT, DkdvShape<D>::OCC) void bwd_dkdv_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  using K = DkdvShape<D>;
  // 64 queries per streamed tile: two 32-query blocks per barrier
  constexpr int BQT = 64, NSB = BQT / 32;
  constexpr int TQT = BQT * C::ROWB, LPT = TQT / (K::NT * 16);
  static_assert(TQT % (K::NT * 16) == 0, "tile loads must divide evenly");
  __shared__ __attribute__((aligned(16))) uint8_t lq0[TQT], ldo0[TQT], lq1[TQT], ldo1[TQT];
  __shared__ __attribute__((aligned(16))) float ll0[BQT], ld0[BQT], ll1[BQT], ld1[BQT];
  // V rows of the work-group's keys (B operand of dP = dO V^T)
  __shared__ __attribute__((aligned(16))) uint8_t lvk[K::BR * C::ROWB];
  auto qbuf = [&](int st) -> uint8_t* { return st == 0 ? lq0 : lq1; };
  auto obuf = [&](int st) -> uint8_t* { return st == 0 ? ldo0 : ldo1; };
  auto lbuf = [&](int st) -> float* { return st == 0 ? ll0 : ll1; };
  auto dbuf = [&](int st) -> float* { return st == 0 ? ld0 : ld1; };

  const int lid = xcd_logical_id(blockIdx.x, p.total_k);
  const bool pair = CAUSAL && p.pair_k;
  const int per_bh = pair ? (p.n_kt + 1) / 2 : p.n_kt;
  const int bh = lid / per_bh;
  const int kt_hi = lid - bh * per_bh;  // causal: the first key blocks see the most queries
  const int kt_lo = CAUSAL ? p.n_kt - 1 - kt_hi : kt_hi;
  const int n_pass = (pair && kt_lo != kt_hi) ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    const int kt = pass == 0 ? kt_hi : kt_lo;
    if (pass > 0) __syncthreads();  // every wave is done with the LDS stages and V rows before refilling
    const int k0 = kt * K::BR;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // lane offsets are recomputed per pass, not held across both
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const size_t head_q = (size_t)bh * p.Nq * D, head_kv = (size_t)bh * p.Nkv * D;
    const uint16_t* __restrict__ qg = p.q + head_q;
    const uint16_t* __restrict__ dog = p.dout + head_q;
    const int kw0 = k0 + 32 * w, kj = kw0 + l32;
    const bool key_ok = kj < p.Nkv;

    // K^T fragments (B operand of S = Q K^T) of this lane's key
    bf16x8 kf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u};
      if (key_ok) a = load16(p.k + head_kv + (size_t)kj * D + ks * 16 + 8 * h);
      kf[ks] = __builtin_bit_cast(bf16x8, a);
    }
    {  // the block's V rows into LDS (rows past N_kv read zeros); visible after the first barrier
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + head_kv + (size_t)k0 * D, (p.Nkv - k0) * C::ROWB);
      constexpr int LPV = K::BR * C::ROWB / (K::NT * 16);
#pragma unroll
      for (int i = 0; i < LPV; ++i) {
        const int r = C::RPL * (w * LPV + i) + lane / C::CH, pc = lane % C::CH;
        load_lds16(rv, r * C::ROWB + 16 * (pc ^ swz_kv<D>(r)), lvk + 1024 * (w * LPV + i));
      }
    }
    const uint8_t* vrow = lvk + 32 * w * C::ROWB;  // this wave's 32 keys
    const float c = p.c;

    // query tiles: causal blocks start at the first query that may see key k0
    const int n_qtiles = (p.Nq + BQT - 1) / BQT;
    const int t0 = CAUSAL ? max(0, k0 - p.off) / BQT : 0;
    const int wave_q_first = kw0 >= p.Nkv ? p.Nq : (CAUSAL ? max(0, kw0 - p.off) : 0);

    f32x16 acck[C::MBD], accv[C::MBD];  // dK^T, dV^T
#pragma unroll
    for (int mbd = 0; mbd < C::MBD; ++mbd) acck[mbd] = accv[mbd] = f32x16{};

    int ld_off[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int r = C::RPL * (w * LPT + i) + lane / C::CH, pc = lane % C::CH;
      ld_off[i] = r * C::ROWB + 16 * (pc ^ swz_kv<D>(r));
    }
    auto load_tile = [&](int t, int stage) {
      const int qr0 = t * BQT;
      const int bytes = (p.Nq - qr0) * C::ROWB;
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + (size_t)qr0 * D, bytes);
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(dog + (size_t)qr0 * D, bytes);
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int blk = 1024 * (w * LPT + i);
        load_lds16(rq, ld_off[i], qbuf(stage) + blk);
        load_lds16(ro, ld_off[i], obuf(stage) + blk);
      }
      if (w == 0 && lane < BQT / 4) {  // LSE and D of the tile's queries (zeros past N_q)
        const size_t e = (size_t)bh * p.Nq + qr0;
        load_lds16(make_rsrc(p.lse + e, (p.Nq - qr0) * 4), 16 * lane, lbuf(stage));
        load_lds16(make_rsrc(p.delta + e, (p.Nq - qr0) * 4), 16 * lane, dbuf(stage));
      }
    };
    int row_off[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) row_off[ks] = l32 * C::ROWB + 16 * ((2 * ks + h) ^ swz_kv<D>(l32));
    int trq[C::MBD][2];
#pragma unroll
    for (int mbd = 0; mbd < C::MBD; ++mbd) {
      trq[mbd][0] = tr_offset<D>(lane, mbd, 0);
      trq[mbd][1] = tr_offset<D>(lane, mbd, 1);
    }

    // one 32-query block at row 32 sb of the tile: C rows are queries qr0 + 8 g + 4 h + (r & 3), g = r / 4;
    // the lane's column is key kj
    auto compute_block = [&](int st, int sb, bool masked, int qr0, bool first, auto&& next) {
      const uint8_t* qb = qbuf(st) + 32 * sb * C::ROWB;
      const uint8_t* ob = obuf(st) + 32 * sb * C::ROWB;
      f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qb + row_off[ks]);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], S, 0, 0, 0);
        const bf16x8 oa = *reinterpret_cast<const bf16x8*>(ob + row_off[ks]);
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(vrow + row_off[ks]);
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vb, dP, 0, 0, 0);
      }
      if (first) next();
      const float* lt = lbuf(st) + 32 * sb;
      const float* dt = dbuf(st) + 32 * sb;
      bf16x8 bs[2], bp[2];  // dS and P, packed for the B operand
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        float xs[8], xp[8];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g = 2 * kc + g2;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + 8 * g + 4 * h);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + 8 * g + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float pr = exp2_hw(fmaf(S[r], c, -l4[e] * kLog2e));
            if (masked && kj > qr0 + 8 * g + 4 * h + e + p.off) pr = 0.f;
            xs[4 * g2 + e] = pr * (dP[r] - d4[e]);
            xp[4 * g2 + e] = pr;
          }
        }
        u32x4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(xs[2 * i], xs[2 * i + 1]);
        bs[kc] = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(xp[2 * i], xp[2 * i + 1]);
        bp[kc] = __builtin_bit_cast(bf16x8, pk);
      }
      // dV^T += dO^T P, then dK^T += Q^T dS (dO^T, Q^T through transposing reads)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int mbd = 0; mbd < C::MBD; ++mbd)
          accv[mbd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(ob + 16 * kc * C::ROWB, trq[mbd]), bp[kc],
                                                              accv[mbd], 0, 0, 0);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int mbd = 0; mbd < C::MBD; ++mbd)
          acck[mbd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(qb + 16 * kc * C::ROWB, trq[mbd]), bs[kc],
                                                              acck[mbd], 0, 0, 0);
    };

    auto tile = [&](auto stage_tag, int t) {
      constexpr int STAGE = decltype(stage_tag)::value;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const bool more = t + 1 < n_qtiles;
      auto next = [&]() {
        if (more) load_tile(t + 1, STAGE ^ 1);
      };
      const int qr0 = t * BQT;
      bool first = true;  // the next tile's loads go out after the first computed block's score MFMAs
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int qb0 = qr0 + 32 * sb;
        if (qb0 + 31 < wave_q_first) continue;  // every query of the block precedes the wave's keys
        compute_block(STAGE, sb, CAUSAL && qb0 < kw0 + 31 - p.off, qb0, first, next);
        first = false;
      }
      if (first) next();
    };

    if (t0 < n_qtiles) load_tile(t0, 0);
    for (int t = t0; t < n_qtiles; t += 2) {
      tile(std::integral_constant<int, 0>{}, t);
      if (t + 1 < n_qtiles) tile(std::integral_constant<int, 1>{}, t + 1);
    }
    __builtin_amdgcn_s_waitcnt(0);  // every load has landed before the work-group ends (no tile: V rows)
    if (key_ok) {
      store_rowT<D>(p.dk + head_kv + (size_t)kj * D, acck, p.scale, h);
      store_rowT<D>(p.dv + head_kv + (size_t)kj * D, accv, 1.f, h);
    }
  }
}

// ------------------------------------------------------------------------------------------------ launch

template <int D, bool CAUSAL>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  using C = BwdCfg<D>;
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<const uint16_t*>(a.o);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.Nq = a.Nq;
  p.Nkv = a.Nkv;
  p.off = a.Nkv - a.Nq;
  p.n_qt = (a.Nq + C::BR - 1) / C::BR;
  p.n_kt = (a.Nkv + DkdvShape<D>::BR - 1) / DkdvShape<D>::BR;
  // pair causal blocks when a grid spans at least two work-groups per compute unit (below that every block
  // runs at once and pairing would only lengthen the longest chain)
  p.pair_q = plan_bwd_dq(a.B, a.H, a.Nq, D, CAUSAL, a.num_cu).paired;
  p.pair_k = plan_bwd_dkdv(a.B, a.H, a.Nkv, D, CAUSAL, a.num_cu).paired;
  p.total_q = a.B * a.H * (p.pair_q ? (p.n_qt + 1) / 2 : p.n_qt);
  p.total_k = a.B * a.H * (p.pair_k ? (p.n_kt + 1) / 2 : p.n_kt);
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(p.total_q), dim3(C::NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(p.total_k), dim3(DkdvShape<D>::NT), 0, s, p);
  return hipGetLastError();
}

LaunchPlan plan_bwd_dq(int B, int H, int Nq, int d, bool causal, int num_cu) {
  LaunchPlan pl;
  pl.kernel = kKernelBwdDq;
  pl.waves = d == 128 ? BwdCfg<128>::NW : BwdCfg<64>::NW;
  pl.rows = d == 128 ? BwdCfg<128>::BR : BwdCfg<64>::BR;
  const int n = (Nq + pl.rows - 1) / pl.rows;
  pl.paired = causal && n >= 2 && (int64_t)B * H * n >= 2 * (int64_t)num_cu;
  pl.groups = (int64_t)B * H * (pl.paired ? (n + 1) / 2 : n);
  return pl;
}

LaunchPlan plan_bwd_dkdv(int B, int H, int Nkv, int d, bool causal, int num_cu) {
  LaunchPlan pl;
  pl.kernel = kKernelBwdDkdv;
  pl.waves = d == 128 ? DkdvShape<128>::NT / 64 : DkdvShape<64>::NT / 64;
  pl.rows = d == 128 ? DkdvShape<128>::BR : DkdvShape<64>::BR;
  const int n = (Nkv + pl.rows - 1) / pl.rows;
  pl.paired = causal && n >= 2 && (int64_t)B * H * n >= 2 * (int64_t)num_cu;
  pl.groups = (int64_t)B * H * (pl.paired ? (n + 1) / 2 : n);
  return pl;
}

int64_t bwd_bf16_grid(int B, int H, int Nq, int Nkv) {
  const int64_t bh = (int64_t)B * H;
  const int64_t a = bh * ((Nq + 127) / 128), b = bh * ((Nkv + 127) / 128);
  return a > b ? a : b;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  if (a.d == 128) return a.causal ? launch_bwd_d<128, true>(a, s) : launch_bwd_d<128, false>(a, s);
  return a.causal ? launch_bwd_d<64, true>(a, s) : launch_bwd_d<64, false>(a, s);
}

}  // namespace fa
