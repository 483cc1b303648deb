// Tiled exact attention forward, fp32 in / fp32 out, fp32 throughout, for gfx950 (MI355X).
//
// Same recurrence as the bf16 kernel (running max m, running denominator l, rescaled output O; see
// "How FlashAttention Works", part 3, of "FlashAttention Explained: How AI Models Process Attention
// Faster and Use Less Memory"), but nothing is rounded below fp32: scores and value sums run on
// v_mfma_f32_32x32x2_f32 and the probabilities enter the value product unrounded.
//
// Layout: S^T = K Q^T as in the bf16 kernel (a lane owns one query column).  Each MFMA contracts two
// d values (one per lane half); the d order is permuted so that a lane reads 4 consecutive floats of
// a K row (and of its Q row) per 16-byte access and feeds them to 4 consecutive MFMAs.  For
// O^T = V^T P^T the probability is the lane's own score register and V is read one float per lane
// from a row-major LDS copy (padded rows against bank conflicts between the two lane halves).
// Grids with fewer work-groups than compute units use prefill_f32_ks_kernel instead, which splits each
// row's keys over the waves of a work-group and merges their partials (below).
#include "common.h"
#include "kernels.h"

namespace fa {

struct PrefillF32Params {
  const float* __restrict__ q;
  const float* __restrict__ k;
  const float* __restrict__ v;
  float* __restrict__ o;
  float* __restrict__ lse;
  int Nq, Nkv, off, n_qt, total;
  float c;
  uint32_t qxor;  // 0x80000000 when scale < 0
};

template <int D, int NW, int BC>
struct F32Cfg {
  static constexpr int BR = NW * 32;
  static constexpr int NT = NW * 64;
  static constexpr int KCH = D / 4;           // 16-byte chunks per row
  static constexpr int CPT = BC * KCH / NT;   // chunks staged per thread (K and V each)
  static constexpr int VSTRIDE = D + 8;       // padded V row (floats)
  static constexpr int MB = BC / 32;
  static constexpr int KS4 = D / 8;           // groups of 4 MFMA k-steps over d
  static constexpr int MBD = D / 32;
  static constexpr int LDS_K = BC * D;
  static constexpr int LDS_V = BC * VSTRIDE;
  static constexpr int LDS_ELEMS = 2 * (LDS_K + LDS_V);
  static_assert(BC * KCH % NT == 0, "staging must divide evenly");
};

// One 32-key tile of a wave's 32 query rows: S^T = K Q^T on fp32 MFMAs (K from `ks`, the swizzled
// row-major tile), mask, online softmax update of (m, l) and O^T += V^T P^T (V one float per lane from the
// padded row-major tile `vs`).  m is in log2 units; l is this lane half's partial row sum.
template <int D, int BC>
__device__ __forceinline__ void f32_tile(const float* ks, const float* vs, int kv0, bool need_mask, int lim,
                                         float c, int h, int l32, const f32x4 (&qf)[D / 8],
                                         f32x16 (&oacc)[D / 32], float& m_run, float& l_run) {
  using C = F32Cfg<D, 4, BC>;
  f32x16 sacc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) sacc[mb] = f32x16{};
#pragma unroll
  for (int g = 0; g < C::KS4; ++g) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const int row = mb * 32 + l32, cc = 2 * g + h;
      const f32x4 kf = *reinterpret_cast<const f32x4*>(ks + (row * C::KCH + (cc ^ (row & 15))) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[i], qf[g][i], sacc[mb], 0, 0, 0);
    }
  }
  if (need_mask) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key > lim) sacc[mb][r] = kNegInf;
      }
  }
  float mx = kNegInf;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mb][r]);
  mx = fmaxf(mx, xor32(mx));
  const float mt = (mx == kNegInf) ? kNegInf : mx * c;
  const float mn = fmaxf(m_run, mt);
  const float alpha = (m_run == kNegInf) ? 0.f : exp2_hw(m_run - mn);
  const float msub = (mn == kNegInf) ? 0.f : mn;
  float rs = 0.f;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float sv = sacc[mb][r];
      float pv = exp2_hw(fmaf(sv, c, -msub));
      if (need_mask) pv = (sv == kNegInf) ? 0.f : pv;
      rs += pv;
      sacc[mb][r] = pv;
    }
  l_run = alpha * l_run + rs;
  m_run = mn;
#pragma unroll
  for (int mbd = 0; mbd < C::MBD; ++mbd) oacc[mbd] *= alpha;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
      for (int mbd = 0; mbd < C::MBD; ++mbd) {
        const float vv = vs[key * C::VSTRIDE + mbd * 32 + l32];
        oacc[mbd] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, sacc[mb][r], oacc[mbd], 0, 0, 0);
      }
    }
}

template <int D, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void prefill_f32_kernel(PrefillF32Params p) {
  using C = F32Cfg<D, NW, BC>;
  __shared__ __attribute__((aligned(16))) float smem[C::LDS_ELEMS];

  const int lid = xcd_logical_id(blockIdx.x, p.total);
  const int bh = lid / p.n_qt;
  int qt = lid - bh * p.n_qt;
  if (CAUSAL) qt = p.n_qt - 1 - qt;
  const int q0 = qt * C::BR;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const size_t head_q = (size_t)bh * p.Nq * D;
  const size_t head_kv = (size_t)bh * p.Nkv * D;
  const float* __restrict__ qg = p.q + head_q;
  const float* __restrict__ kg = p.k + head_kv;
  const float* __restrict__ vg = p.v + head_kv;
  const int qw0 = q0 + w * 32;
  const int qi = qw0 + l32;

  // Q^T fragments: for step group g, lane holds q[qi][8g + 4h .. +3]
  f32x4 qf[C::KS4];
#pragma unroll
  for (int g = 0; g < C::KS4; ++g) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < p.Nq) x = load16(qg + (size_t)qi * D + 8 * g + 4 * h);
    x ^= p.qxor;
    qf[g] = __builtin_bit_cast(f32x4, x);
  }

  int kv_end = p.Nkv;
  if (CAUSAL) kv_end = min(p.Nkv, q0 + C::BR + p.off);
  const int n_tiles = (kv_end + BC - 1) / BC;
  const int wave_kv_end = CAUSAL ? min(p.Nkv, qw0 + 32 + p.off) : p.Nkv;

  f32x16 oacc[C::MBD];
#pragma unroll
  for (int mbd = 0; mbd < C::MBD; ++mbd) oacc[mbd] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  u32x4 kst[C::CPT], vst[C::CPT];
  auto load_tile = [&](int t) {
    const int kv0 = t * BC;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int x = tid + i * C::NT, row = x / C::KCH, c = x % C::KCH, key = kv0 + row;
      const bool ok = key < p.Nkv;
      kst[i] = ok ? load16(kg + (size_t)key * D + c * 4) : u32x4{0u, 0u, 0u, 0u};
      vst[i] = ok ? load16(vg + (size_t)key * D + c * 4) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int stage) {
    float* ks = smem + stage * (C::LDS_K + C::LDS_V);
    float* vs = ks + C::LDS_K;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int x = tid + i * C::NT, row = x / C::KCH, c = x % C::KCH;
      store16(ks + (row * C::KCH + (c ^ (row & 15))) * 4, kst[i]);
      store16(vs + row * C::VSTRIDE + c * 4, vst[i]);
    }
  };

  auto compute_tile = [&](int kv0, int stage) {
    const float* ks = smem + stage * (C::LDS_K + C::LDS_V);
    const float* vs = ks + C::LDS_K;
    const bool need_mask = (kv0 + BC > p.Nkv) || (CAUSAL && kv0 + BC - 1 > qw0 + p.off);
    const int lim = CAUSAL ? min(p.Nkv - 1, qi + p.off) : p.Nkv - 1;
    f32_tile<D, BC>(ks, vs, kv0, need_mask, lim, p.c, h, l32, qf, oacc, m_run, l_run);
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

  const float lt = l_run + xor32(l_run);
  const float inv = 1.f / lt;
  if (qi < p.Nq) {
    float* orow = p.o + head_q + (size_t)qi * D;
#pragma unroll
    for (int mbd = 0; mbd < C::MBD; ++mbd)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 val = {oacc[mbd][4 * g4 + 0] * inv, oacc[mbd][4 * g4 + 1] * inv, oacc[mbd][4 * g4 + 2] * inv,
                     oacc[mbd][4 * g4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + mbd * 32 + 8 * g4 + 4 * h) = val;
      }
    if (h == 0 && p.lse) p.lse[(size_t)bh * p.Nq + qi] = (m_run + log2_hw(lt)) * kLn2;
  }
}

// Small grids (fewer work-groups than compute units, such as one head of 256 queries): one work-group
// per 32 query rows, whose KW waves walk interleaved 32-key tiles of the rows' key range (tile t goes to
// wave t mod KW), each staging its own tile in its own LDS slice, and at the end merge their (m, l, O)
// partials by their log-sum-exp, as the split-KV decode combine does.  Each wave's serial chain of fp32
// MFMAs is then KW times shorter than one wave walking the whole row.
template <int D, int KW, int BC, bool CAUSAL>
__global__ __launch_bounds__(KW * 64) void prefill_f32_ks_kernel(PrefillF32Params p) {
  using C = F32Cfg<D, 4, BC>;
  constexpr int WREG = C::LDS_K + C::LDS_V;  // floats of one wave's slice
  constexpr int CPL = BC * C::KCH / 64;      // 16-byte chunks of a tile per lane (K and V each)
  static_assert(BC * C::KCH % 64 == 0, "staging must divide evenly");
  static_assert(2 * KW * 32 + KW * 32 * D <= KW * WREG, "the merge must fit in the tile slices");
  __shared__ __attribute__((aligned(16))) float smem[KW * WREG];

  const int lid = xcd_logical_id(blockIdx.x, p.total);
  const int bh = lid / p.n_qt;
  int qt = lid - bh * p.n_qt;
  if (CAUSAL) qt = p.n_qt - 1 - qt;
  const int q0 = qt * 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int qi = q0 + l32;
  const size_t head_q = (size_t)bh * p.Nq * D;
  const size_t head_kv = (size_t)bh * p.Nkv * D;
  const float* __restrict__ kg = p.k + head_kv;
  const float* __restrict__ vg = p.v + head_kv;

  f32x4 qf[C::KS4];
#pragma unroll
  for (int g = 0; g < C::KS4; ++g) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < p.Nq) x = load16(p.q + head_q + (size_t)qi * D + 8 * g + 4 * h);
    x ^= p.qxor;
    qf[g] = __builtin_bit_cast(f32x4, x);
  }
  const int kv_end = CAUSAL ? min(p.Nkv, q0 + 32 + p.off) : p.Nkv;
  const int n_tiles = (kv_end + BC - 1) / BC;
  const int lim = CAUSAL ? min(p.Nkv - 1, qi + p.off) : p.Nkv - 1;

  f32x16 oacc[C::MBD];
#pragma unroll
  for (int mbd = 0; mbd < C::MBD; ++mbd) oacc[mbd] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  float* ks = smem + w * WREG;
  float* vs = ks + C::LDS_K;
  for (int t = w; t < n_tiles; t += KW) {
    const int kv0 = t * BC;
    // the wave's own slice: LDS operations of one wave take effect in order, so no barrier is needed
    // between this tile's stores, its reads and the next tile's stores
    // K and V requested together when both fit in registers (d = 64: 16 chunks per lane), else K first
    constexpr bool KV_TOGETHER = CPL <= 8;
    u32x4 sk[CPL], sv[KV_TOGETHER ? CPL : 1];
    auto load_rows = [&](const float* src, u32x4 (&dst)[CPL]) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int x = lane + 64 * i, row = x / C::KCH, cc = x % C::KCH, key = kv0 + row;
        dst[i] = key < p.Nkv ? load16(src + (size_t)key * D + cc * 4) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto store_k = [&](const u32x4 (&src)[CPL]) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int x = lane + 64 * i, row = x / C::KCH, cc = x % C::KCH;
        store16(ks + (row * C::KCH + (cc ^ (row & 15))) * 4, src[i]);
      }
    };
    auto store_v = [&](const u32x4 (&src)[CPL]) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int x = lane + 64 * i, row = x / C::KCH, cc = x % C::KCH;
        store16(vs + row * C::VSTRIDE + cc * 4, src[i]);
      }
    };
    load_rows(kg, sk);
    if constexpr (KV_TOGETHER) {
      load_rows(vg, sv);
      store_k(sk);
      store_v(sv);
    } else {
      store_k(sk);
      load_rows(vg, sk);
      store_v(sk);
    }
    const bool need_mask = (kv0 + BC > p.Nkv) || (CAUSAL && kv0 + BC - 1 > q0 + p.off);
    f32_tile<D, BC>(ks, vs, kv0, need_mask, lim, p.c, h, l32, qf, oacc, m_run, l_run);
  }

  // merge the waves' partials: m (log2 units) and l per row, unnormalised O per row and column
  const float lw = l_run + xor32(l_run);
  __syncthreads();  // every wave is done with its tile slice
  float* cm = smem;
  float* cl = cm + KW * 32;
  float* co = cl + KW * 32;
  if (h == 0) {
    cm[w * 32 + l32] = m_run;
    cl[w * 32 + l32] = lw;
  }
#pragma unroll
  for (int mbd = 0; mbd < C::MBD; ++mbd)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 val = {oacc[mbd][4 * g4 + 0], oacc[mbd][4 * g4 + 1], oacc[mbd][4 * g4 + 2], oacc[mbd][4 * g4 + 3]};
      *reinterpret_cast<f32x4*>(co + (w * 32 + l32) * D + mbd * 32 + 8 * g4 + 4 * h) = val;
    }
  __syncthreads();
  for (int idx = tid; idx < 32 * D; idx += KW * 64) {
    const int r = idx / D, dd = idx - r * D, row = q0 + r;
    if (row >= p.Nq) break;  // rows are in order: every later index is past N_q too
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < KW; ++u) mx = fmaxf(mx, cm[u * 32 + r]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int u = 0; u < KW; ++u) {
      const float mu = cm[u * 32 + r];
      const float wt = mu == kNegInf ? 0.f : exp2_hw(mu - mx);  // a wave with no tile of these rows
      num += wt * co[(u * 32 + r) * D + dd];
      den += wt * cl[u * 32 + r];
    }
    p.o[head_q + (size_t)row * D + dd] = num / den;
    if (dd == 0 && p.lse) p.lse[(size_t)bh * p.Nq + row] = (mx + log2_hw(den)) * kLn2;
  }
}

namespace {
constexpr int kNWf = 4;
constexpr int kBCf = 32;
}  // namespace

int64_t prefill_f32_grid(int B, int H, int Nq, int) {
  const int br = kNWf * 32;
  return (int64_t)B * H * ((Nq + br - 1) / br);
}

template <int D, bool CAUSAL>
static hipError_t launch_f32_d(const PrefillArgs& a, hipStream_t s) {
  using C = F32Cfg<D, kNWf, kBCf>;
  PrefillF32Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<float*>(a.o);
  p.lse = a.lse;
  p.Nq = a.Nq;
  p.Nkv = a.Nkv;
  p.off = a.Nkv - a.Nq;
  p.n_qt = (a.Nq + C::BR - 1) / C::BR;
  p.total = a.B * a.H * p.n_qt;
  p.c = fabsf(a.scale) * kLog2e;
  p.qxor = a.scale < 0.f ? 0x80000000u : 0u;
  if (plan_prefill_f32(a.B, a.H, a.Nq, D, a.num_cu).kernel == kKernelF32KeySplit) {
    constexpr int KW = D == 64 ? 8 : 4;
    p.n_qt = (a.Nq + 31) / 32;
    p.total = a.B * a.H * p.n_qt;
    hipLaunchKernelGGL((prefill_f32_ks_kernel<D, KW, kBCf, CAUSAL>), dim3(p.total), dim3(KW * 64), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_f32_kernel<D, kNWf, kBCf, CAUSAL>), dim3(p.total), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

LaunchPlan plan_prefill_f32(int B, int H, int Nq, int d, int num_cu) {
  LaunchPlan pl;
  const int64_t rows_grid = prefill_f32_grid(B, H, Nq, d);
  // fewer work-groups than compute units: split each row's keys over the waves of a 32-row work-group
  if (rows_grid < num_cu) {
    pl.kernel = kKernelF32KeySplit;
    pl.waves = d == 64 ? 8 : 4;
    pl.rows = 32;
    pl.groups = (int64_t)B * H * ((Nq + 31) / 32);
  } else {
    pl.kernel = kKernelF32Rows;
    pl.waves = kNWf;
    pl.rows = kNWf * 32;
    pl.groups = rows_grid;
  }
  return pl;
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  if (a.d == 128) return a.causal ? launch_f32_d<128, true>(a, s) : launch_f32_d<128, false>(a, s);
  return a.causal ? launch_f32_d<64, true>(a, s) : launch_f32_d<64, false>(a, s);
}

}  // namespace fa
