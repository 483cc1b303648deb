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
// are non-temporal (they do not displace reusable lines; +7% HBM throughput measured against plain loads).  The range is processed in
// chunks of up to kChunk keys: (A) scores q.k with v_dot2_f32_bf16 and a reduction over the d/8
// lanes of the row, kept in LDS; (B) chunk max and exponentials 2^(s*c - m) with a work-group
// reduction, and the running (m, l) update; (C) the value sum, each lane accumulating 8 output
// columns over its keys in fp32.  Chunks after the first rescale the running sums by 2^(m_old - m).
// The per-group partial outputs are summed through LDS at the end.
#include "common.h"
#include "kernels.h"

namespace fa {

namespace {
constexpr int kDecThreads = 512;
constexpr int kChunk = 1024;
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
#pragma unroll 8
    for (int j = grp; j < n; j += KPI) {
      const u32x4 kv = load16_nt(kg + (size_t)(cb + j) * D);
      float part = dot8_bf16(qv, kv);
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m);
      if (sl == 0) sc[j] = part * p.c;
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

// One work-group of d threads per (b, h): M = max_s lse_s, w_s = exp(lse_s - M),
// o = sum w_s O_s / sum w_s (rounded to bf16), lse = M + ln sum w_s.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ ws_o,
                                                           const float* __restrict__ ws_lse,
                                                           uint16_t* __restrict__ o, float* __restrict__ lse, int S) {
  const int bh = blockIdx.x, t = threadIdx.x;
  const float* __restrict__ L = ws_lse + (size_t)bh * S;
  const float* __restrict__ Os = ws_o + (size_t)bh * S * D;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, L[s]);
  float sw = 0.f, acc = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ls = L[s];
    const float wgt = (ls == kNegInf) ? 0.f : exp2_hw((ls - M) * kLog2e);
    sw += wgt;
    acc = fmaf(wgt, Os[(size_t)s * D + t], acc);
  }
  const float r = acc / sw;
  const __bf16 b = (__bf16)r;
  o[(size_t)bh * D + t] = __builtin_bit_cast(uint16_t, b);
  if (t == 0 && lse) lse[bh] = M + log2_hw(sw) * kLn2;
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

hipError_t launch_decode_combine_bf16(const CombineArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.B * a.H));
  uint16_t* o = static_cast<uint16_t*>(a.o);
  if (a.d == 128)
    hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(128), 0, s, a.ws_o, a.ws_lse, o, a.lse, a.splits);
  else
    hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(64), 0, s, a.ws_o, a.ws_lse, o, a.lse, a.splits);
  return hipGetLastError();
}

}  // namespace fa
