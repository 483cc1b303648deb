// Measurement probes (declared in include/fa_probe.h): the read-stream bandwidth the HBM actually
// delivers to a plain streaming kernel, and the shader clock under dense matrix-core load.  They put the
// attention kernels' figures in context (a decode kernel is read against what a plain streaming read reaches, a
// prefill kernel against the clock the chip holds under MFMA load); they are not part of the attention
// path and share no code with it.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "common.h"
#include "fa_probe.h"

namespace fa {

namespace {

// Read of n16 16-byte words with the non-temporal policy (read once, not kept in the caches): work-group g
// streams the contiguous span [g * per, (g + 1) * per) of words, per = ceil(n16 / groups), as steps of
// four coalesced 8 KB loads in flight per group (thread t reads words 512 u + t of the step, u = 0..3),
// then the words of the span's last partial step one at a time.  Each thread folds what it read into
// one word so the loads stay live; the fold is stored per thread.
__global__ __launch_bounds__(512) void read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = beg + threadIdx.x;
  for (; i + 3 * 512 < end; i += 4 * 512) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + 512);
    const u32x4 d = __builtin_nontemporal_load(src + i + 1024);
    const u32x4 e = __builtin_nontemporal_load(src + i + 1536);
    acc ^= (a ^ b) ^ (d ^ e);
  }
  for (; i < end; i += 512) acc ^= __builtin_nontemporal_load(src + i);
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Dense bf16 MFMA work on operands that change every instruction (eight different pseudo-random register
// sets in rotation, so the datapath toggles as it does on real data), with the shader clock counter
// (s_memtime) and the constant 100 MHz counter (s_memrealtime) read before and after by each work-group.
__global__ __launch_bounds__(256) void clock_probe_kernel(unsigned long long* __restrict__ out, int iters) {
  const uint32_t lane = threadIdx.x;
  uint32_t x = 0x9e3779b9u * (lane + 1) ^ (blockIdx.x * 0x85ebca6bu);
  auto next = [&]() {  // xorshift32
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
  };
  // bf16 values in [1, 2) with random mantissas and signs: finite, no overflow over the loop
  auto rnd8 = [&]() {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t r = next();
      w[i] = ((r & 0x807f807fu) | 0x3f803f80u);
    }
    return __builtin_bit_cast(bf16x8, w);
  };
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = rnd8();
    b[i] = rnd8();
  }
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  // eight iterations per trip so that every register index is a compile-time value
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + r) & 7], acc[i & 3], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (threadIdx.x == 0) {
    unsigned long long* o = out + 5 * (size_t)blockIdx.x;
    o[0] = t0;
    o[1] = r0;
    o[2] = t1;
    o[3] = r1;
    o[4] = (unsigned long long)(s != s);  // 0 unless the sums went NaN (keeps the MFMAs live)
  }
}

}  // namespace

}  // namespace fa

extern "C" {

int fa_probe_read_bandwidth(const void* buf, size_t bytes, void* sink, size_t sink_bytes, int groups, void* stream) {
  if (!buf || !sink || bytes < 16 || (reinterpret_cast<uintptr_t>(buf) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return 1;
  if (groups < 1 || groups > (1 << 20) || sink_bytes < (size_t)groups * 512 * 4) return 1;
  if (hipGetLastError() != hipSuccess) return 4;  // an error from earlier work: reported, nothing launched
  hipLaunchKernelGGL(fa::read_probe_kernel, dim3(groups), dim3(512), 0, (hipStream_t)stream,
                     static_cast<const fa::u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int fa_probe_clock(unsigned long long* out, size_t out_words, int groups, int iters, void* stream) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 7) || groups < 1 || groups > (1 << 20) || iters < 1 ||
      out_words < (size_t)groups * 5)
    return 1;
  if (hipGetLastError() != hipSuccess) return 4;
  hipLaunchKernelGGL(fa::clock_probe_kernel, dim3(groups), dim3(256), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
