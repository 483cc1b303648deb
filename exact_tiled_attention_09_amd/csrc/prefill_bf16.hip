// Tiled exact attention forward, bf16 in / bf16 out, fp32 accumulation, for gfx950 (MI355X).
//
// Method: the Q/K/V tiling with a running row maximum m, a running denominator l and a rescaled
// partial output O ("FlashAttention Explained: How AI Models Process Attention Faster and Use Less
// Memory", "How FlashAttention Works", parts 1-3; "Flash Attention Explained: Same Maths, Far Less
// Memory", "The idea: never materialise the matrix").  Per key tile j and query row i:
//   m_new = max(m, max_j s_ij * c),  alpha = 2^(m - m_new),  p_ij = 2^(s_ij * c - m_new),
//   l = alpha * l + sum_j p_ij,      O = alpha * O + sum_j p_ij v_j,
// with c = |scale| * log2(e) (exp2 with log2(e) folded into the scale is the same exponential); at
// the end O / l and LSE = ln2 * (m + log2 l).  The score tile lives only in registers.
//
// gfx950 mapping (one work-group per (batch*head, query tile), NW waves, NB*32 query rows per wave):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K is the A operand
//    (read from LDS), Q^T the B operand (held in VGPRs for the whole kernel).  In the 32x32 result
//    a lane holds one query column and 16 keys, so lane l and lane l^32 together own query l%32:
//    row max / row sum are in-lane reductions plus one exchange with lane l^32.
//  * O^T = V^T P^T on the same instruction: P^T is the B operand taken straight from the lane's own
//    score registers (keys are contracted in the order the score layout gives them), V^T the A
//    operand, read from an LDS copy of V stored transposed with the matching key order.  The
//    transpose happens while staging: each thread loads a 4-key x 8-d block (four 16-byte global
//    loads) and writes eight 8-byte LDS rows after v_perm_b32 byte shuffles.
//  * K and V^T tiles are double-buffered in LDS (the next tile's global loads are in flight while
//    the current tile is computed); 16-byte LDS chunks are XOR-swizzled per row against bank conflicts.
//  * Causal tiles above the diagonal are never loaded; a wave skips the math of a tile that is fully
//    masked for its rows; only diagonal and ragged-tail tiles evaluate the mask.
//  * Work-group ids are remapped so each XCD walks contiguous (head, tile) ranges, heaviest causal
//    tiles first.
#include "common.h"
#include "kernels.h"

namespace fa {

struct PrefillParams {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  uint16_t* __restrict__ o;
  float* __restrict__ lse;
  int Nq, Nkv, off, n_qt, total;
  float c;        // |scale| * log2(e)
  uint32_t qxor;  // 0x80008000 when scale < 0: q is negated on load (exact) so that c >= 0
};

template <int D, int NB, int NW, int BC>
struct Bf16Cfg {
  static constexpr int BR = NW * NB * 32;  // query rows per work-group
  static constexpr int NT = NW * 64;       // threads
  static constexpr int KCH = D / 8;        // 16-byte chunks per K row
  static constexpr int VCH = BC / 8;       // 16-byte chunks per V^T row
  static constexpr int KCPT = BC * KCH / NT;   // K chunks staged per thread
  static constexpr int KPT = BC * D / (8 * NT);  // keys per thread in the V staging (4 or 2)
  static constexpr int MB = BC / 32;       // 32-key blocks per tile
  static constexpr int KS = D / 16;        // MFMA k-steps over d
  static constexpr int MBD = D / 32;       // 32-wide d blocks
  static constexpr int KC = BC / 16;       // 16-key chunks contracted by one PV MFMA
  static constexpr int LDS_K = BC * D;     // bf16 elements per stage
  static constexpr int LDS_V = D * BC;
  static constexpr int LDS_ELEMS = 2 * (LDS_K + LDS_V);
  static_assert(KPT == 2 || KPT == 4, "V staging handles 2 or 4 keys per thread");
  static_assert(BC * KCH % NT == 0, "K staging must divide evenly");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shapes");
};

// XOR swizzles of the 16-byte chunk index within a row (see the bank analysis in the design notes).
template <int D>
__device__ __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int BC>
__device__ __forceinline__ int swz_v(int d) { return BC == 128 ? (d & 15) : ((d >> 1) & 7); }

template <int D, int NB, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(PrefillParams p) {
  using C = Bf16Cfg<D, NB, NW, BC>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];

  const int lid = xcd_logical_id(blockIdx.x, p.total);
  const int bh = lid / p.n_qt;
  int qt = lid - bh * p.n_qt;
  if (CAUSAL) qt = p.n_qt - 1 - qt;  // heaviest query tiles first
  const int q0 = qt * C::BR;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const size_t head_q = (size_t)bh * p.Nq * D;
  const size_t head_kv = (size_t)bh * p.Nkv * D;
  const uint16_t* __restrict__ qg = p.q + head_q;
  const uint16_t* __restrict__ kg = p.k + head_kv;
  const uint16_t* __restrict__ vg = p.v + head_kv;
  const int qw0 = q0 + w * NB * 32;  // first query row of this wave

  // Q^T fragments: lane holds query qw0 + nb*32 + l32, d = ks*16 + 8h .. +7.
  bf16x8 qf[NB][C::KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int qi = qw0 + nb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi < p.Nq) x = load16(qg + (size_t)qi * D + ks * 16 + 8 * h);
      x ^= p.qxor;
      qf[nb][ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  int kv_end = p.Nkv;
  if (CAUSAL) kv_end = min(p.Nkv, q0 + C::BR + p.off);
  const int n_tiles = (kv_end + BC - 1) / BC;
  const int wave_kv_end = CAUSAL ? min(p.Nkv, qw0 + NB * 32 + p.off) : p.Nkv;

  f32x16 oacc[NB][C::MBD];
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.f;
#pragma unroll
    for (int mbd = 0; mbd < C::MBD; ++mbd) oacc[nb][mbd] = f32x16{};
  }

  u32x4 kst[C::KCPT];
  u32x4 vst[C::KPT];
  const int v_cd = tid % (D / 8), v_g = tid / (D / 8);

  auto load_tile = [&](int t) {
    const int kv0 = t * BC;
#pragma unroll
    for (int i = 0; i < C::KCPT; ++i) {
      const int x = tid + i * C::NT, row = x / C::KCH, c = x % C::KCH, key = kv0 + row;
      kst[i] = key < p.Nkv ? load16(kg + (size_t)key * D + c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < C::KPT; ++e) {
      const int key = kv0 + v_g * C::KPT + e;
      vst[e] = key < p.Nkv ? load16(vg + (size_t)key * D + v_cd * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  auto store_tile = [&](int stage) {
    uint16_t* ks = smem + stage * (C::LDS_K + C::LDS_V);
    uint16_t* vs = ks + C::LDS_K;
#pragma unroll
    for (int i = 0; i < C::KCPT; ++i) {
      const int x = tid + i * C::NT, row = x / C::KCH, c = x % C::KCH;
      store16(ks + (row * C::KCH + (c ^ swz_k<D>(row))) * 8, kst[i]);
    }
    // V^T: keys of each 16-key chunk are stored in the order the score layout contracts them,
    // [0-3, 8-11, 4-7, 12-15], so lane half h later reads its 8 keys as one 16-byte chunk.
    const int kb = v_g * C::KPT;
    const int kc = kb >> 4, e = kb & 15, lg = e >> 2;
    const int cc = 2 * kc + (lg & 1), elem = 4 * (lg >> 1) + (e & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int dd = 0; dd < 2; ++dd) {
        const int d = v_cd * 8 + 2 * j + dd;
        uint16_t* dst = vs + d * BC + (cc ^ swz_v<BC>(d)) * 8 + elem;
        if constexpr (C::KPT == 4) {
          u32x2 val;
          val[0] = dd ? perm_hi(vst[1][j], vst[0][j]) : perm_lo(vst[1][j], vst[0][j]);
          val[1] = dd ? perm_hi(vst[3][j], vst[2][j]) : perm_lo(vst[3][j], vst[2][j]);
          *reinterpret_cast<u32x2*>(dst) = val;
        } else {
          *reinterpret_cast<uint32_t*>(dst) = dd ? perm_hi(vst[1][j], vst[0][j]) : perm_lo(vst[1][j], vst[0][j]);
        }
      }
    }
  };

  auto compute_tile = [&](int kv0, int stage) {
    const uint16_t* ks = smem + stage * (C::LDS_K + C::LDS_V);
    const uint16_t* vs = ks + C::LDS_K;
    f32x16 sacc[C::MB][NB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[mb][nb] = f32x16{};
    // S^T = K Q^T
#pragma unroll
    for (int kstep = 0; kstep < C::KS; ++kstep) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int row = mb * 32 + l32, c = 2 * kstep + h;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (row * C::KCH + (c ^ swz_k<D>(row))) * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sacc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nb][kstep], sacc[mb][nb], 0, 0, 0);
      }
    }
    // mask (diagonal and ragged tail only), online softmax
    const bool need_mask = (kv0 + BC > p.Nkv) || (CAUSAL && kv0 + BC - 1 > qw0 + p.off);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (need_mask) {
        const int qi = qw0 + nb * 32 + l32;
        const int lim = CAUSAL ? min(p.Nkv - 1, qi + p.off) : p.Nkv - 1;  // last allowed key
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key > lim) sacc[mb][nb][r] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mb][nb][r]);
      mx = fmaxf(mx, xor32(mx));
      const float mt = (mx == kNegInf) ? kNegInf : mx * p.c;
      const float mn = fmaxf(m_run[nb], mt);
      const float alpha = (m_run[nb] == kNegInf) ? 0.f : exp2_hw(m_run[nb] - mn);
      const float msub = (mn == kNegInf) ? 0.f : mn;
      float rs = 0.f;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s = sacc[mb][nb][r];
          float pv = exp2_hw(fmaf(s, p.c, -msub));
          if (need_mask) pv = (s == kNegInf) ? 0.f : pv;
          rs += pv;
          sacc[mb][nb][r] = pv;
        }
      l_run[nb] = alpha * l_run[nb] + rs;
      m_run[nb] = mn;
#pragma unroll
      for (int mbd = 0; mbd < C::MBD; ++mbd) oacc[nb][mbd] *= alpha;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      bf16x8 pf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x16& s = sacc[kc >> 1][nb];
        const int r0 = 8 * (kc & 1);
        u32x4 pk;
        pk[0] = pack_bf16x2(s[r0 + 0], s[r0 + 1]);
        pk[1] = pack_bf16x2(s[r0 + 2], s[r0 + 3]);
        pk[2] = pack_bf16x2(s[r0 + 4], s[r0 + 5]);
        pk[3] = pack_bf16x2(s[r0 + 6], s[r0 + 7]);
        pf[nb] = __builtin_bit_cast(bf16x8, pk);
      }
#pragma unroll
      for (int mbd = 0; mbd < C::MBD; ++mbd) {
        const int d = mbd * 32 + l32, cc = 2 * kc + h;
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs + d * BC + (cc ^ swz_v<BC>(d)) * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          oacc[nb][mbd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nb], oacc[nb][mbd], 0, 0, 0);
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const int kv0 = t * BC;
    if (kv0 < wave_kv_end) compute_tile(kv0, stage);
    if (t + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // epilogue: O / l rounded to bf16 (nearest even), LSE = ln2 * (m + log2 l)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = l_run[nb] + xor32(l_run[nb]);
    const float inv = 1.f / lt;
    const int qi = qw0 + nb * 32 + l32;
    if (qi < p.Nq) {
      uint16_t* orow = p.o + head_q + (size_t)qi * D;
#pragma unroll
      for (int mbd = 0; mbd < C::MBD; ++mbd)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& a = oacc[nb][mbd];
          u32x2 val;
          val[0] = pack_bf16x2(a[4 * g4 + 0] * inv, a[4 * g4 + 1] * inv);
          val[1] = pack_bf16x2(a[4 * g4 + 2] * inv, a[4 * g4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + mbd * 32 + 8 * g4 + 4 * h) = val;
        }
      if (h == 0 && p.lse) p.lse[(size_t)bh * p.Nq + qi] = (m_run[nb] + log2_hw(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------------------------- launch

namespace {
constexpr int kNW = 4;
constexpr int kBC = 64;
template <int D>
constexpr int nb_for() { return 1; }
}  // namespace

int64_t prefill_bf16_grid(int B, int H, int Nq, int d) {
  const int br = kNW * 32 * (d == 128 ? nb_for<128>() : nb_for<64>());
  return (int64_t)B * H * ((Nq + br - 1) / br);
}

template <int D, bool CAUSAL>
static hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
  constexpr int NB = nb_for<D>();
  using C = Bf16Cfg<D, NB, kNW, kBC>;
  PrefillParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.Nq = a.Nq;
  p.Nkv = a.Nkv;
  p.off = a.Nkv - a.Nq;
  p.n_qt = (a.Nq + C::BR - 1) / C::BR;
  p.total = a.B * a.H * p.n_qt;
  p.c = fabsf(a.scale) * kLog2e;
  p.qxor = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NB, kNW, kBC, CAUSAL>), dim3(p.total), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  if (a.d == 128) return a.causal ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
  return a.causal ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
}

}  // namespace fa
