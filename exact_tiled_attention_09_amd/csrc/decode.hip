// Split-KV decode for gfx950: one query per sequence against its cached keys and values.
//
// During decode the score matrix is a single row per (batch, head) ("Flash Attention Explained: Same
// Maths, Far Less Memory", "Where you actually feel it"), so there is nothing for the matrix cores to
// do (one flop per byte) and the kernel is an HBM stream of K and V.  The keys of a row are cut into
// S contiguous ranges; one work-group per (b, h, s) computes the normalised partial output O_s and
// its log-sum-exp over its range, and a second kernel merges the S partials by their LSE weights.
//
// Split kernel (512 threads): a key row of d bf16 is read by d/8 lanes with one 16-byte load each,
// so a wave reads 64*16 contiguous-row bytes per load instruction.  K and V are read once, so the loads
// are non-temporal (they do not displace reusable lines; +7% HBM throughput measured against plain
// loads).  The range is processed in chunks of up to kChunk keys: (A) scores q.k with v_dot2_f32_bf16
// and a DPP reduction over the d/8 lanes of the row, kept in LDS; (B) chunk max and exponentials 2^(s*c - m) with a work-group
// reduction, and the running (m, l) update; (C) the value sum, each lane accumulating 8 output
// columns over its keys in fp32.  Chunks after the first rescale the running sums by 2^(m_old - m).
// The per-group partial outputs are summed through LDS at the end.
#include "common.h"
#include "kernels.h"

namespace fa {

namespace {
constexpr int kDecThreads = 512;
constexpr int kChunk = 1024;
// K rows loaded per lane before their scores are reduced (16: +6% on B64 H32 N_kv8192 d128, at four
// waves per SIMD instead of eight)
constexpr int kScoreBatch = 16;
}  // namespace

struct DecodeParams {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  float* __restrict__ ws_o;
  float* __restrict__ ws_lse;
  int Nkv, S, per_split;
  float c;
  uint32_t qxor;
};

// 16-byte load that streams past the caches (each K / V byte is read once).
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Dot product of 8 bf16 pairs with v_dot2_f32_bf16 (fp32 accumulation).  The pairs are taken from
// whole-vector casts: casting single dwords of the vector to bf16x2 was folded by the compiler into
// four uses of the first dword.
__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b) {
  const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 xa = {x[2 * i], x[2 * i + 1]}, ya = {y[2 * i], y[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(xa, ya, acc, false);
  }
  return acc;
}

// Sum over the LPR lanes that share a key row (aligned groups of 8 or 16 lanes), in every lane of the
// group, with DPP lane moves folded into the adds (no LDS-crossbar permutes):
//   16 lanes: rotate by 8 and by 4 within the row, then swap within pairs of the quad and within pairs;
//    8 lanes: mirror within the half row, mirror within the quad, then swap within pairs.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRor8 = 0x128, kDppRor4 = 0x124, kDppHalfMirror = 0x141;
constexpr int kDppQuadMirror = 0x1B;  // quad_perm [3,2,1,0]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LPR == 8 || LPR == 16, "key rows span 8 or 16 lanes");
  if (LPR == 16) {
    x += dpp_mov<kDppRor8>(x);
    x += dpp_mov<kDppRor4>(x);
    x += dpp_mov<kDppQuadSwap2>(x);
  } else {
    x += dpp_mov<kDppHalfMirror>(x);
    x += dpp_mov<kDppQuadMirror>(x);
  }
  x += dpp_mov<kDppQuadSwap1>(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeParams p) {
  constexpr int LPR = D / 8;                  // lanes per key row
  constexpr int KPI = kDecThreads / LPR;      // keys per work-group iteration
  constexpr int NWV = kDecThreads / 64;
  __shared__ float sc[kChunk];
  __shared__ float red[KPI * D];
  __shared__ float wred[NWV];

  const int bhs = blockIdx.x;
  const int s = bhs % p.S;
  const int bh = bhs / p.S;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sl = tid % LPR, grp = tid / LPR;
  const int k0 = min(s * p.per_split, p.Nkv);
  const int k1 = min(k0 + p.per_split, p.Nkv);
  float* __restrict__ out_o = p.ws_o + (size_t)bhs * D;

  if (k1 <= k0) {  // empty range: zero weight in the combine
    if (tid < D) out_o[tid] = 0.f;
    if (tid == 0) p.ws_lse[bhs] = kNegInf;
    return;
  }

  const uint16_t* __restrict__ kg = p.k + (size_t)bh * p.Nkv * D + 8 * sl;
  const uint16_t* __restrict__ vg = p.v + (size_t)bh * p.Nkv * D + 8 * sl;
  u32x4 qv = load16(p.q + (size_t)bh * D + 8 * sl);
  qv ^= p.qxor;

  float m_run = kNegInf, l_run = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  for (int cb = k0; cb < k1; cb += kChunk) {
    const int n = min(kChunk, k1 - cb);
    // (A) scores, in log2 units
    for (int j0 = grp; j0 < n; j0 += kScoreBatch * KPI) {
      // the batch's loads first: the row reductions are cross-lane operations, which keep the compiler
      // from unrolling a loop with a run-time trip count, so the batching is written out
      u32x4 kv[kScoreBatch];
#pragma unroll
      for (int u = 0; u < kScoreBatch; ++u) {
        const int j = j0 + u * KPI;
        kv[u] = j < n ? load16_nt(kg + (size_t)(cb + j) * D) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kScoreBatch; ++u) {
        const int j = j0 + u * KPI;
        const float part = row_sum<LPR>(dot8_bf16(qv, kv[u]));
        if (sl == 0 && j < n) sc[j] = part * p.c;
      }
    }
    __syncthreads();
    // (B) chunk max, exponentials, chunk sum
    float mx = kNegInf;
    for (int j = tid; j < n; j += kDecThreads) mx = fmaxf(mx, sc[j]);
    mx = wave_max(mx);
    if (lane == 0) wred[w] = mx;
    __syncthreads();
    mx = wred[0];
#pragma unroll
    for (int i = 1; i < NWV; ++i) mx = fmaxf(mx, wred[i]);
    const float mn = fmaxf(m_run, mx);
    const float alpha = (m_run == kNegInf) ? 0.f : exp2_hw(m_run - mn);
    float ps = 0.f;
    for (int j = tid; j < n; j += kDecThreads) {
      const float e = exp2_hw(sc[j] - mn);
      sc[j] = e;
      ps += e;
    }
    ps = wave_sum(ps);
    __syncthreads();  // every wave has read wred (max) and written its exponentials
    if (lane == 0) wred[w] = ps;
    __syncthreads();
    ps = 0.f;
#pragma unroll
    for (int i = 0; i < NWV; ++i) ps += wred[i];
    l_run = alpha * l_run + ps;
    m_run = mn;
    // (C) value sum
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
#pragma unroll 8
    for (int j = grp; j < n; j += KPI) {
      const u32x4 vv = load16_nt(vg + (size_t)(cb + j) * D);
      const float pj = sc[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = fmaf(pj, bf16lo_to_f32(vv[i]), o[2 * i]);
        o[2 * i + 1] = fmaf(pj, bf16hi_to_f32(vv[i]), o[2 * i + 1]);
      }
    }
    __syncthreads();  // sc and wred are reused by the next chunk
  }

  // sum the per-group partial outputs
#pragma unroll
  for (int i = 0; i < 8; ++i) red[grp * D + 8 * sl + i] = o[i];
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll 8
    for (int g = 0; g < KPI; ++g) acc += red[g * D + tid];
    out_o[tid] = acc / l_run;
  }
  if (tid == 0) p.ws_lse[bhs] = (m_run + log2_hw(l_run)) * kLn2;
}

// Paged KV cache ("Paged Attention: Fixing the KV Cache Memory Problem", listed among the related posts of
// "Flash Attention Explained: Speed From Memory Movement"): the cache is a pool of fixed-size pages
// [num_pages, H_kv, P, d] and a per-sequence block table maps token t to page table[b][t / P], row t % P.
// One work-group per (b, h_kv, s) serves the G = H / H_kv query heads that share key/value head h_kv, so
// each K and V row is streamed once for all G of them.  The S ranges of a sequence split its own length
// (read on the device), so ragged batches stay balanced.  At the start of every chunk the table entries
// it covers are staged in LDS (entries outside the pool become -1: their tokens are absent, read nothing
// and get weight 0); a key row is then one LDS read, an address computation and the 16-byte loads of the
// contiguous-cache kernel above.  Scores of the G heads are kept in LDS side by side (G * 4 KB).
struct PagedParams {
  const uint16_t* __restrict__ q;     // [B, H, D]
  const uint16_t* __restrict__ kp;    // [num_pages, H_kv, P, D]
  const uint16_t* __restrict__ vp;
  const int* __restrict__ table;      // [B, max_blocks]
  const int* __restrict__ seq_lens;   // [B]
  float* __restrict__ ws_o;           // [B * H, S, D]
  float* __restrict__ ws_lse;         // [B * H, S]
  int Hkv, S, num_pages, max_blocks, lg_page;
  float c;
  uint32_t qxor;
};

template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_paged_kernel(PagedParams p) {
  constexpr int LPR = D / 8;
  constexpr int KPI = kDecThreads / LPR;
  constexpr int NWV = kDecThreads / 64;
  constexpr int CH = kChunk;
  __shared__ float sc[G][CH];
  __shared__ int ptab[CH + 1];
  __shared__ float red[KPI * D];
  __shared__ float wred[G][NWV];

  const int bks = blockIdx.x;
  const int s = bks % p.S;
  const int bk = bks / p.S;  // b * H_kv + h_kv
  const int b = bk / p.Hkv, hkv = bk - b * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sl = tid % LPR, grp = tid / LPR;
  const int lg = p.lg_page, pmask = (1 << lg) - 1;
  const int len = min(max(p.seq_lens[b], 0), p.max_blocks << lg);
  const int per = (len + p.S - 1) / p.S;
  const int k0 = min(s * per, len);
  const int k1 = min(k0 + per, len);
  const size_t row0 = (size_t)b * p.Hkv * G + (size_t)hkv * G;  // first query row (b, h_kv * G)

  const int* __restrict__ tab = p.table + (size_t)b * p.max_blocks;
  const uint16_t* __restrict__ kg = p.kp + (size_t)hkv * ((size_t)D << lg) + 8 * sl;
  const uint16_t* __restrict__ vg = p.vp + (size_t)hkv * ((size_t)D << lg) + 8 * sl;
  const size_t page_elems = (size_t)p.Hkv * ((size_t)D << lg);

  u32x4 qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    qv[g] = load16(p.q + (row0 + g) * D + 8 * sl);
    qv[g] ^= p.qxor;
  }
  float m_run[G], l_run[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = kNegInf;
    l_run[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[g][i] = 0.f;
  }

  for (int cb = k0; cb < k1; cb += CH) {
    const int n = min(CH, k1 - cb);
    const int pg0 = cb >> lg;
    const int npg = ((cb + n - 1) >> lg) - pg0 + 1;
    for (int i = tid; i < npg; i += kDecThreads) {
      const int e = tab[pg0 + i];
      ptab[i] = (e >= 0 && e < p.num_pages) ? e : -1;
    }
    __syncthreads();
    // (A) scores of the G query heads, in log2 units (-inf for absent tokens)
    // K rows per lane in flight: 8 for one head (16, as in the contiguous kernel, measured 7% slower here
    // with the page lookups), 4 for grouped heads (registers grow with G)
    constexpr int NB = G == 1 ? 8 : 4;
    for (int j0 = grp; j0 < n; j0 += NB * KPI) {
      u32x4 kv[NB];
      bool here[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int j = j0 + u * KPI;
        const int t = cb + j;
        const int pg = j < n ? ptab[(t >> lg) - pg0] : -1;
        here[u] = pg >= 0;
        kv[u] = here[u] ? load16_nt(kg + (size_t)pg * page_elems + (size_t)(t & pmask) * D) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int j = j0 + u * KPI;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float part = row_sum<LPR>(dot8_bf16(qv[g], kv[u]));
          if (sl == 0 && j < n) sc[g][j] = here[u] ? part * p.c : kNegInf;
        }
      }
    }
    __syncthreads();
    // (B) per head: chunk max, exponentials, chunk sum, running (m, l) update
    float alpha[G];
    {
      float mx[G];
#pragma unroll
      for (int g = 0; g < G; ++g) mx[g] = kNegInf;
      for (int j = tid; j < n; j += kDecThreads) {
#pragma unroll
        for (int g = 0; g < G; ++g) mx[g] = fmaxf(mx[g], sc[g][j]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        mx[g] = wave_max(mx[g]);
        if (lane == 0) wred[g][w] = mx[g];
      }
      __syncthreads();
      float ms[G], ps[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float m = wred[g][0];
#pragma unroll
        for (int i = 1; i < NWV; ++i) m = fmaxf(m, wred[g][i]);
        const float mn = fmaxf(m_run[g], m);
        alpha[g] = (m_run[g] == kNegInf) ? 0.f : exp2_hw(m_run[g] - mn);
        ms[g] = (mn == kNegInf) ? 0.f : mn;  // all scores -inf so far: every weight is 0
        m_run[g] = mn;
        ps[g] = 0.f;
      }
      for (int j = tid; j < n; j += kDecThreads) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float e = exp2_hw(sc[g][j] - ms[g]);
          sc[g][j] = e;
          ps[g] += e;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) ps[g] = wave_sum(ps[g]);
      __syncthreads();  // every wave has read wred (max) and written its exponentials
      if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) wred[g][w] = ps[g];
      }
      __syncthreads();
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < NWV; ++i) t += wred[g][i];
        l_run[g] = alpha[g] * l_run[g] + t;
      }
    }
    // (C) value sums
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[g][i] *= alpha[g];
    }
#pragma unroll 4
    for (int j = grp; j < n; j += KPI) {
      const int t = cb + j;
      const int pg = ptab[(t >> lg) - pg0];
      if (pg < 0) continue;
      const u32x4 vv = load16_nt(vg + (size_t)pg * page_elems + (size_t)(t & pmask) * D);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pj = sc[g][j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[g][2 * i] = fmaf(pj, bf16lo_to_f32(vv[i]), o[g][2 * i]);
          o[g][2 * i + 1] = fmaf(pj, bf16hi_to_f32(vv[i]), o[g][2 * i + 1]);
        }
      }
    }
    __syncthreads();  // sc, ptab and wred are reused by the next chunk
  }

  // per head: sum the per-group partial outputs and write the normalised partial and its LSE
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const size_t row = (row0 + g) * p.S + s;
#pragma unroll
    for (int i = 0; i < 8; ++i) red[grp * D + 8 * sl + i] = o[g][i];
    __syncthreads();
    if (tid < D) {
      float acc = 0.f;
#pragma unroll 8
      for (int q = 0; q < KPI; ++q) acc += red[q * D + tid];
      p.ws_o[row * D + tid] = l_run[g] > 0.f ? acc / l_run[g] : 0.f;
    }
    if (tid == 0) p.ws_lse[row] = l_run[g] > 0.f ? (m_run[g] + log2_hw(l_run[g])) * kLn2 : kNegInf;
    __syncthreads();  // red is reused by the next head
  }
}

// Per row (one (b, h), or one query row of a split prefill): M = max_s lse_s, w_s = exp(lse_s - M),
// o = sum w_s O_s / sum w_s (rounded to bf16), lse = M + ln sum w_s.  Each thread owns four consecutive
// d of one row (16-byte loads of the fp32 partials, an 8-byte store of the bf16 result), so a 256-thread
// work-group covers 256 / (D / 4) rows; the loop over ranges is unrolled so several loads are in flight.
// Per element the operations and their order are those of a plain loop over s.
constexpr int kCombineThreads = 256;
template <int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(const float* __restrict__ ws_o,
                                                                        const float* __restrict__ ws_lse,
                                                                        uint16_t* __restrict__ o,
                                                                        float* __restrict__ lse, int64_t rows, int S) {
  constexpr int TPR = D / 4, RPW = kCombineThreads / TPR;  // threads per row, rows per work-group
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
  const int d0 = 4 * (threadIdx.x % TPR);
  if (row >= rows) return;
  const float* __restrict__ L = ws_lse + (size_t)row * S;
  const float* __restrict__ Os = ws_o + (size_t)row * S * D + d0;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, L[s]);
  float sw = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float ls = L[s];
    const float wgt = (ls == kNegInf) ? 0.f : exp2_hw((ls - M) * kLog2e);
    sw += wgt;
    const f32x4 v = *reinterpret_cast<const f32x4*>(Os + (size_t)s * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(wgt, v[e], acc[e]);
  }
  // sw == 0 only when every range was empty (a paged sequence with no tokens): O = 0, LSE = -inf
  u32x2 out;
#pragma unroll
  for (int e = 0; e < 2; ++e)
    out[e] = pack_bf16x2(sw > 0.f ? acc[2 * e] / sw : 0.f, sw > 0.f ? acc[2 * e + 1] / sw : 0.f);
  *reinterpret_cast<u32x2*>(o + (size_t)row * D + d0) = out;
  if (d0 == 0 && lse) lse[row] = sw > 0.f ? M + log2_hw(sw) * kLn2 : kNegInf;
}

hipError_t launch_decode_split_bf16(const DecodeArgs& a, hipStream_t s) {
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.ws_o = a.ws_o;
  p.ws_lse = a.ws_lse;
  p.Nkv = a.Nkv;
  p.S = a.splits;
  p.per_split = (a.Nkv + a.splits - 1) / a.splits;
  p.c = fabsf(a.scale) * kLog2e;
  p.qxor = a.scale < 0.f ? 0x80008000u : 0u;
  const dim3 grid((unsigned)((int64_t)a.B * a.H * a.splits));
  if (a.d == 128)
    hipLaunchKernelGGL(decode_split_kernel<128>, grid, dim3(kDecThreads), 0, s, p);
  else
    hipLaunchKernelGGL(decode_split_kernel<64>, grid, dim3(kDecThreads), 0, s, p);
  return hipGetLastError();
}

namespace {
template <int D>
hipError_t launch_paged_d(const PagedParams& p, int G, dim3 grid, hipStream_t s) {
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_paged_kernel<D, 1>), grid, dim3(kDecThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_paged_kernel<D, 2>), grid, dim3(kDecThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_paged_kernel<D, 4>), grid, dim3(kDecThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_paged_kernel<D, 8>), grid, dim3(kDecThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_paged_bf16(const PagedDecodeArgs& a, hipStream_t s) {
  PagedParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.kp = static_cast<const uint16_t*>(a.k_pages);
  p.vp = static_cast<const uint16_t*>(a.v_pages);
  p.table = a.block_table;
  p.seq_lens = a.seq_lens;
  p.ws_o = a.ws_o;
  p.ws_lse = a.ws_lse;
  p.Hkv = a.Hkv;
  p.S = a.splits;
  p.num_pages = a.num_pages;
  p.max_blocks = a.max_blocks;
  int lg = 0;
  while ((1 << lg) < a.page_size) ++lg;
  p.lg_page = lg;
  p.c = fabsf(a.scale) * kLog2e;
  p.qxor = a.scale < 0.f ? 0x80008000u : 0u;
  const dim3 grid((unsigned)((int64_t)a.B * a.Hkv * a.splits));
  const int G = a.H / a.Hkv;
  return a.d == 128 ? launch_paged_d<128>(p, G, grid, s) : launch_paged_d<64>(p, G, grid, s);
}

hipError_t launch_decode_combine_bf16(const CombineArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H;
  const int rpw = kCombineThreads / (a.d / 4);
  const dim3 grid((unsigned)((rows + rpw - 1) / rpw));
  uint16_t* o = static_cast<uint16_t*>(a.o);
  if (a.d == 128)
    hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(kCombineThreads), 0, s, a.ws_o, a.ws_lse, o, a.lse,
                       rows, a.splits);
  else
    hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(kCombineThreads), 0, s, a.ws_o, a.ws_lse, o, a.lse,
                       rows, a.splits);
  return hipGetLastError();
}

}  // namespace fa
