// C ABI of libfa (declared in include/fa.h): argument validation and dispatch to the gfx950 kernels.
//
// Every check happens on the host before any HIP call, so a rejected request launches nothing and
// leaves the outputs untouched.  Unsupported requests are errors, never a slower fallback path.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <climits>

#include "common.h"
#include "fa.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

fa_status ok() { return FA_OK; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range span(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// n1*n2*... in 64 bits with overflow detection; false if any factor is negative or the product overflows.
bool mul_ok(int64_t& out, std::initializer_list<int64_t> xs) {
  int64_t r = 1;
  for (int64_t x : xs) {
    if (x < 0) return false;
    if (x != 0 && r > INT64_MAX / x) return false;
    r *= x;
  }
  out = r;
  return true;
}

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // per tensor; far beyond any device memory

fa_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// An error left pending on this thread by earlier work is reported as such (and nothing is launched):
// clearing it silently would hide the caller's failure, and launching on top of it would report it as ours.
fa_status take_pending(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return ok();
  return fail(FA_ERR_DEVICE, "%s: an error from earlier work was pending on this thread: %s (nothing was launched)",
              what, hipGetErrorString(e));
}

fa_status check_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q, int N_kv,
                    int d, float scale, int causal, fa_dtype dtype, size_t* esz) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (B < 1 || H < 1 || N_q < 1 || N_kv < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H, N_q, N_kv must be >= 1 (got %d, %d, %d, %d)", B, H, N_q, N_kv);
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head size d=%d is not built (supported: 64, 128)", d);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  if (causal && N_q > N_kv)
    return fail(FA_ERR_INVALID_ARG, "causal attention needs N_q <= N_kv (got N_q=%d, N_kv=%d)", N_q, N_kv);
  *esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
  int64_t nq_el, nkv_el;
  if (!mul_ok(nq_el, {B, H, N_q, d}) || !mul_ok(nkv_el, {B, H, N_kv, d}) || nq_el > kMaxElems || nkv_el > kMaxElems)
    return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  // the bf16 kernel addresses one head's K and V through 32-bit buffer byte ranges
  if (dtype == FA_DTYPE_BF16 && (int64_t)N_kv * d * 2 > INT_MAX)
    return fail(FA_ERR_UNSUPPORTED, "bf16 prefill supports N_kv * d * 2 <= 2^31 - 1 bytes per head (got N_kv=%d, d=%d)",
                N_kv, d);
  const int64_t grid = dtype == FA_DTYPE_BF16 ? fa::prefill_bf16_grid(B, H, N_q, d, 0) : fa::prefill_f32_grid(B, H, N_q, d);
  if (grid > INT_MAX) return fail(FA_ERR_INVALID_ARG, "launch grid too large (%lld work-groups)", (long long)grid);
  const Range rq = span(q, nq_el * *esz), rk = span(k, nkv_el * *esz), rv = span(v, nkv_el * *esz);
  const Range ro = span(o, nq_el * *esz);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv)) return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (lse) {
    const Range rl = span(lse, (size_t)B * H * N_q * 4);
    if (overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv) || overlap(rl, ro))
      return fail(FA_ERR_INVALID_ARG, "lse overlaps another tensor");
  }
  return FA_OK;
}

int auto_splits(int B, int H, int N_kv, int num_cu) {
  // Enough work-groups to cover the CUs eight times (decode is bound by the bytes in flight), without
  // splits shorter than 256 keys.
  const int64_t bh = (int64_t)B * H;
  int64_t s = (8 * (int64_t)num_cu + bh - 1) / bh;
  const int64_t max_by_len = (N_kv + 255) / 256;
  if (s > max_by_len) s = max_by_len;
  if (s < 1) s = 1;
  return (int)s;
}

fa_status check_decode_sizes(int B, int H, int N_kv, int d, int num_splits, int* S) {
  if (B < 1 || H < 1 || N_kv < 1) return fail(FA_ERR_INVALID_ARG, "B, H, N_kv must be >= 1");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head size d=%d is not built (supported: 64, 128)", d);
  if (num_splits < 0 || num_splits > N_kv)
    return fail(FA_ERR_INVALID_ARG, "num_splits must be in [0, N_kv] (got %d)", num_splits);
  *S = num_splits == 0 ? auto_splits(B, H, N_kv, fa::planning_cu_count()) : num_splits;
  int64_t el;
  if (!mul_ok(el, {B, H, N_kv, d}) || el > kMaxElems) return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  int64_t g;
  if (!mul_ok(g, {B, H, *S}) || g > INT_MAX) return fail(FA_ERR_INVALID_ARG, "launch grid too large");
  return FA_OK;
}

size_t ws_bytes(int B, int H, int d, int S) { return (size_t)B * H * S * (d + 1) * sizeof(float); }

fa_status check_workspace(const void* ws, size_t have, size_t need) {
  if (!ws) return fail(FA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 16)) return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  if (have < need) return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return FA_OK;
}

}  // namespace

namespace fa {

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();  // no usable device: nothing can be launched on this thread anyway
    return 0;
  }
  const int have = cache[dev].load(std::memory_order_relaxed);
  if (have > 0) return have;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 0;
  }
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int planning_cu_count() {
  const int n = device_cu_count();
  return n > 0 ? n : kDefaultNumCu;
}

}  // namespace fa

namespace {

int fwd_split_auto(int B, int H, int N_q, int N_kv, int num_cu) {
  // The split work-groups are bound by matrix-core work, not by bytes in flight: one round of the two
  // that are resident per compute unit is enough (on a 1000-query chunk against 8192 keys, 2 splits and
  // 4 splits each won on some GPUs by up to 7%; 3 and 8 lost 10-20% to uneven rounds and the fixed
  // costs of short splits); no split is made shorter than 512 keys.
  const int64_t units = (int64_t)B * H * ((N_q + 127) / 128);
  int64_t s = (2 * (int64_t)num_cu + units - 1) / units;
  const int64_t max_by_len = (N_kv + 511) / 512;
  if (s > max_by_len) s = max_by_len;
  if (s < 1) s = 1;
  return (int)s;
}

}  // namespace

// Scratch of the allocation-free decode: one copy per GPU, in the library's code object, so no call ever
// allocates.  Host code uses only the address looked up per device below, never the array's name (on the
// host that name is a stand-in, not a device address).
constexpr size_t kNoAllocScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];

// The current device's copy of `scratch`, looked up on the first call on that device with the device
// current.  Two threads racing here look up and store the same address.
fa_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // reported here; not left pending for the next call
    return fail(FA_ERR_DEVICE, "fa_decode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(FA_ERR_DEVICE, "fa_decode_noalloc: device %d beyond the %d the library tracks", dev, kMaxScratchDevices);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(FA_ERR_DEVICE, "fa_decode_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q, int N_kv,
                 int d, float scale, int causal, void* stream, fa_dtype dtype) {
  size_t esz = 0;
  const fa_status st = check_fwd(q, k, v, o, lse, B, H, N_q, N_kv, d, scale, causal, dtype, &esz);
  if (st != FA_OK) return st;
  fa::PrefillArgs a{q, k, v, o, lse, B, H, N_q, N_kv, d, scale, causal != 0};
  a.num_cu = fa::planning_cu_count();
  const fa_status pend = take_pending("fa_fwd");
  if (pend != FA_OK) return pend;
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_prefill_bf16(a, (hipStream_t)stream)
                                              : fa::launch_prefill_f32(a, (hipStream_t)stream);
  return device_status(e, "fa_fwd launch");
}

fa_status fa_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q,
                      int N_kv, int d, float scale, int causal, void* stream) {
  return fa_fwd(q, k, v, o, lse, B, H, N_q, N_kv, d, scale, causal, stream, FA_DTYPE_BF16);
}

fa_status fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q,
                     int N_kv, int d, float scale, int causal, void* stream) {
  return fa_fwd(q, k, v, o, lse, B, H, N_q, N_kv, d, scale, causal, stream, FA_DTYPE_F32);
}

int fa_decode_num_splits(int B, int H, int N_kv, int d, int num_splits) {
  int S = 0;
  if (check_decode_sizes(B, H, N_kv, d, num_splits, &S) != FA_OK) return 0;
  return S;
}

size_t fa_decode_workspace_bytes(int B, int H, int N_kv, int d, int num_splits) {
  int S = 0;
  if (check_decode_sizes(B, H, N_kv, d, num_splits, &S) != FA_OK) return 0;
  return ws_bytes(B, H, d, S);
}

fa_status fa_decode_split(const void* q, const void* k, const void* v, int B, int H, int N_kv, int d, float scale,
                          int num_splits, void* workspace, size_t workspace_bytes, void* stream, fa_dtype dtype) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!q || !k || !v) return fail(FA_ERR_INVALID_ARG, "q, k and v must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
  int S = 0;
  fa_status st = check_decode_sizes(B, H, N_kv, d, num_splits, &S);
  if (st != FA_OK) return st;
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  if (dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "decode is built for bf16 only");
  const size_t need = ws_bytes(B, H, d, S);
  st = check_workspace(workspace, workspace_bytes, need);
  if (st != FA_OK) return st;
  const size_t kv_bytes = (size_t)B * H * N_kv * d * 2, q_bytes = (size_t)B * H * d * 2;
  const Range rw = span(workspace, need);
  if (overlap(rw, span(q, q_bytes)) || overlap(rw, span(k, kv_bytes)) || overlap(rw, span(v, kv_bytes)))
    return fail(FA_ERR_INVALID_ARG, "workspace overlaps an input");
  float* ws_o = static_cast<float*>(workspace);
  fa::DecodeArgs a{q, k, v, B, H, N_kv, d, scale, S, ws_o, ws_o + (size_t)B * H * S * d};
  const fa_status pend = take_pending("fa_decode_split");
  if (pend != FA_OK) return pend;
  return device_status(fa::launch_decode_split_bf16(a, (hipStream_t)stream), "fa_decode split launch");
}

fa_status fa_decode_combine(const void* workspace, size_t workspace_bytes, void* o, float* lse, int B, int H, int d,
                            int num_splits, void* stream, fa_dtype dtype) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!o) return fail(FA_ERR_INVALID_ARG, "o must be non-NULL");
  if (!aligned(o, 16)) return fail(FA_ERR_INVALID_ARG, "o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (B < 1 || H < 1) return fail(FA_ERR_INVALID_ARG, "B, H must be >= 1");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head size d=%d is not built (supported: 64, 128)", d);
  if (num_splits < 1) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 1 for the combine (got %d)", num_splits);
  int64_t g;
  if (!mul_ok(g, {B, H, num_splits, d + 1}) || g > kMaxElems) return fail(FA_ERR_INVALID_ARG, "sizes overflow");
  if (dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "decode is built for bf16 only");
  const size_t need = ws_bytes(B, H, d, num_splits);
  fa_status st = check_workspace(workspace, workspace_bytes, need);
  if (st != FA_OK) return st;
  const Range rw = span(workspace, need), ro = span(o, (size_t)B * H * d * 2);
  if (overlap(rw, ro)) return fail(FA_ERR_INVALID_ARG, "o overlaps the workspace");
  if (lse) {
    const Range rl = span(lse, (size_t)B * H * 4);
    if (overlap(rl, rw) || overlap(rl, ro)) return fail(FA_ERR_INVALID_ARG, "lse overlaps another buffer");
  }
  const float* ws_o = static_cast<const float*>(workspace);
  fa::CombineArgs a{ws_o, ws_o + (size_t)B * H * num_splits * d, o, lse, B, H, d, num_splits};
  const fa_status pend = take_pending("fa_decode_combine");
  if (pend != FA_OK) return pend;
  return device_status(fa::launch_decode_combine_bf16(a, (hipStream_t)stream), "fa_decode combine launch");
}

fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_kv, int d,
                    float scale, int num_splits, void* workspace, size_t workspace_bytes, void* stream,
                    fa_dtype dtype) {
  // Validate both halves before launching either, so a rejected call enqueues nothing.
  if (!o) return fail(FA_ERR_INVALID_ARG, "o must be non-NULL");
  if (!aligned(o, 16)) return fail(FA_ERR_INVALID_ARG, "o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!q || !k || !v) return fail(FA_ERR_INVALID_ARG, "q, k and v must be non-NULL");
  int S = 0;
  fa_status st = check_decode_sizes(B, H, N_kv, d, num_splits, &S);
  if (st != FA_OK) return st;
  const size_t q_bytes = (size_t)B * H * d * 2, kv_bytes = (size_t)B * H * N_kv * d * 2;
  const Range ro = span(o, q_bytes);
  if (overlap(ro, span(q, q_bytes)) || overlap(ro, span(k, kv_bytes)) || overlap(ro, span(v, kv_bytes)))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (lse) {
    const Range rl = span(lse, (size_t)B * H * 4);
    if (overlap(rl, span(q, q_bytes)) || overlap(rl, span(k, kv_bytes)) || overlap(rl, span(v, kv_bytes)) ||
        overlap(rl, ro))
      return fail(FA_ERR_INVALID_ARG, "lse overlaps another tensor");
  }
  if (workspace) {
    const Range rw = span(workspace, ws_bytes(B, H, d, S));
    if (overlap(rw, ro) || (lse && overlap(rw, span(lse, (size_t)B * H * 4))))
      return fail(FA_ERR_INVALID_ARG, "workspace overlaps an output");
  }
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  if (dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "decode is built for bf16 only");
  st = check_workspace(workspace, workspace_bytes, ws_bytes(B, H, d, S));
  if (st != FA_OK) return st;
  st = fa_decode_split(q, k, v, B, H, N_kv, d, scale, S, workspace, workspace_bytes, stream, dtype);
  if (st != FA_OK) return st;
  return fa_decode_combine(workspace, workspace_bytes, o, lse, B, H, d, S, stream, dtype);
}

fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                            int N_kv, int d, float scale, int num_splits, void* stream, fa_dtype dtype) {
  int S = 0;
  fa_status st = check_decode_sizes(B, H, N_kv, d, num_splits, &S);
  if (st != FA_OK) return st;
  const size_t need = ws_bytes(B, H, d, S);
  if (need > kNoAllocScratchBytes)
    return fail(FA_ERR_WORKSPACE,
                "fa_decode_noalloc: the partials need %zu bytes, the built-in scratch holds %zu (B*H*S*(d+1)*4 must "
                "fit; call fa_decode with a workspace instead)",
                need, kNoAllocScratchBytes);
  const fa_status pend = take_pending("fa_decode_noalloc");
  if (pend != FA_OK) return pend;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != FA_OK) return st;
  return fa_decode(q, k, v, o, lse, B, H, N_kv, d, scale, S, ws, kNoAllocScratchBytes, stream, dtype);
}

int fa_fwd_split_num_splits(int B, int H, int N_q, int N_kv, int d) {
  if (B < 1 || H < 1 || N_q < 1 || N_kv < 1 || (d != 64 && d != 128)) return 0;
  return fwd_split_auto(B, H, N_q, N_kv, fa::planning_cu_count());
}

size_t fa_fwd_split_workspace_bytes(int B, int H, int N_q, int d, int num_splits) {
  int64_t n;
  if (B < 1 || H < 1 || N_q < 1 || num_splits < 1 || (d != 64 && d != 128) ||
      !mul_ok(n, {B, H, N_q, num_splits, d + 1, 4}) || n > kMaxElems)
    return 0;
  return (size_t)n;
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q,
                       int N_kv, int d, float scale, int causal, int num_splits, void* workspace,
                       size_t workspace_bytes, void* stream, fa_dtype dtype) {
  size_t esz = 0;
  fa_status st = check_fwd(q, k, v, o, lse, B, H, N_q, N_kv, d, scale, causal, dtype, &esz);
  if (st != FA_OK) return st;
  if (dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "the split-KV forward is built for bf16 only");
  if (num_splits < 1 || num_splits > N_kv)
    return fail(FA_ERR_INVALID_ARG, "num_splits must be in [1, N_kv] (got %d)", num_splits);
  if (fa::prefill_bf16_grid(B, H, N_q, d, num_splits) > INT_MAX ||
      (int64_t)B * H * N_q > INT_MAX)
    return fail(FA_ERR_INVALID_ARG, "launch grid too large");
  const size_t need = fa_fwd_split_workspace_bytes(B, H, N_q, d, num_splits);
  if (need == 0) return fail(FA_ERR_INVALID_ARG, "workspace size overflows");
  st = check_workspace(workspace, workspace_bytes, need);
  if (st != FA_OK) return st;
  const size_t nq_b = (size_t)B * H * N_q * d * 2, nkv_b = (size_t)B * H * N_kv * d * 2;
  const Range rw = span(workspace, need);
  if (overlap(rw, span(q, nq_b)) || overlap(rw, span(k, nkv_b)) || overlap(rw, span(v, nkv_b)) ||
      overlap(rw, span(o, nq_b)) || (lse && overlap(rw, span(lse, (size_t)B * H * N_q * 4))))
    return fail(FA_ERR_INVALID_ARG, "workspace overlaps a tensor");
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o + (size_t)B * H * N_q * num_splits * d;
  fa::PrefillArgs a{q, k, v, o, lse, B, H, N_q, N_kv, d, scale, causal != 0, num_splits, ws_o, ws_lse};
  a.num_cu = fa::planning_cu_count();
  const fa_status pend = take_pending("fa_fwd_split");
  if (pend != FA_OK) return pend;
  hipError_t e = fa::launch_prefill_bf16(a, (hipStream_t)stream);
  if (e != hipSuccess) return device_status(e, "fa_fwd_split launch");
  fa::CombineArgs cmb{ws_o, ws_lse, o, lse, B * H * N_q, 1, d, num_splits};
  return device_status(fa::launch_decode_combine_bf16(cmb, (hipStream_t)stream), "fa_fwd_split combine launch");
}

int fa_decode_gqa_num_splits(int B, int H, int H_kv, int N_kv, int d, int num_splits) {
  if (H_kv < 1 || H < H_kv || H % H_kv != 0) return 0;
  return fa_decode_num_splits(B, H_kv, N_kv, d, num_splits);
}

size_t fa_decode_gqa_workspace_bytes(int B, int H, int H_kv, int N_kv, int d, int num_splits) {
  const int S = fa_decode_gqa_num_splits(B, H, H_kv, N_kv, d, num_splits);
  if (S < 1) return 0;
  return fa_fwd_split_workspace_bytes(B, H_kv, H / H_kv, d, S);
}

fa_status fa_decode_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                        int N_kv, int d, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                        void* stream, fa_dtype dtype) {
  if (H_kv < 1 || H < 1 || H % H_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "H must be a positive multiple of H_kv (got H=%d, H_kv=%d)", H, H_kv);
  int S = 0;
  fa_status st = check_decode_sizes(B, H_kv, N_kv, d, num_splits, &S);
  if (st != FA_OK) return st;
  // the G = H / H_kv query heads of a key/value head are the query rows of one forward over its cache
  return fa_fwd_split(q, k, v, o, lse, B, H_kv, H / H_kv, N_kv, d, scale, 0, S, workspace, workspace_bytes, stream,
                      dtype);
}

int fa_decode_paged_num_splits(int B, int H_kv, int max_seq_len, int d, int num_splits) {
  if (max_seq_len < 1) return 0;
  return fa_decode_num_splits(B, H_kv, max_seq_len, d, num_splits);
}

size_t fa_decode_paged_workspace_bytes(int B, int H, int H_kv, int max_seq_len, int d, int num_splits) {
  if (H_kv < 1 || H < H_kv || H % H_kv != 0) return 0;
  const int S = fa_decode_paged_num_splits(B, H_kv, max_seq_len, d, num_splits);
  if (S < 1) return 0;
  int64_t n;
  if (!mul_ok(n, {B, H, S, d + 1, 4}) || n > kMaxElems) return 0;
  return (size_t)n;
}

fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                          const int* seq_lens, void* o, float* lse, int B, int H, int H_kv, int num_pages,
                          int page_size, int max_blocks, int d, float scale, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream, fa_dtype dtype) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !o)
    return fail(FA_ERR_INVALID_ARG, "q, k_pages, v_pages, block_table, seq_lens and o must be non-NULL");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k_pages, v_pages and o must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
    return fail(FA_ERR_INVALID_ARG, "block_table, seq_lens and lse must be 4-byte aligned");
  if (B < 1 || H < 1 || H_kv < 1 || num_pages < 1 || max_blocks < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H, H_kv, num_pages and max_blocks must be >= 1");
  if (H % H_kv != 0) return fail(FA_ERR_INVALID_ARG, "H must be a multiple of H_kv (got H=%d, H_kv=%d)", H, H_kv);
  if (page_size < 1 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
    return fail(FA_ERR_INVALID_ARG, "page_size must be a power of two in [1, 2^20] (got %d)", page_size);
  // Grouped heads on pages of >= 8 tokens go through the matrix-core split kernel (any group size); one
  // query head per key/value head, or smaller pages, through the vector kernel (groups of 1, 2, 4, 8).
  const int G = H / H_kv;
  const bool mfma_path = G >= 2 && page_size >= 8;
  if (!mfma_path && G != 1 && G != 2 && G != 4 && G != 8)
    return fail(FA_ERR_UNSUPPORTED, "paged decode with page_size < 8 is built for H / H_kv in {1, 2, 4, 8} (got %d)",
                G);
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head size d=%d is not built (supported: 64, 128)", d);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  int64_t max_len, pool_el, q_el, tab_el;
  // 2^30 keeps every token index of the kernel, range ends and chunk steps included, inside int
  if (!mul_ok(max_len, {max_blocks, page_size}) || max_len > (1 << 30))
    return fail(FA_ERR_INVALID_ARG, "max_blocks * page_size must be <= 2^30 (got %d * %d)", max_blocks, page_size);
  if (!mul_ok(pool_el, {num_pages, H_kv, page_size, d}) || pool_el > kMaxElems || !mul_ok(q_el, {B, H, d}) ||
      !mul_ok(tab_el, {B, max_blocks}) || tab_el > kMaxElems)
    return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  if (num_splits < 0 || num_splits > max_len)
    return fail(FA_ERR_INVALID_ARG, "num_splits must be in [0, max_blocks * page_size] (got %d)", num_splits);
  const int S = fa_decode_paged_num_splits(B, H_kv, (int)max_len, d, num_splits);
  int64_t grid;
  if (S < 1 || !mul_ok(grid, {B, H_kv, S}) || grid > INT_MAX ||
      (mfma_path && fa::prefill_bf16_grid(B, H_kv, G, d, S) > INT_MAX))
    return fail(FA_ERR_INVALID_ARG, "launch grid too large");
  const Range rq = span(q, q_el * 2), rk = span(k_pages, pool_el * 2), rv = span(v_pages, pool_el * 2);
  const Range rt = span(block_table, tab_el * 4), rs = span(seq_lens, (size_t)B * 4);
  const Range ro = span(o, q_el * 2);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(ro, rt) || overlap(ro, rs))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  const Range rl = span(lse, lse ? (size_t)B * H * 4 : 0);
  if (lse && (overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv) || overlap(rl, rt) || overlap(rl, rs) ||
              overlap(rl, ro)))
    return fail(FA_ERR_INVALID_ARG, "lse overlaps another tensor");
  if (dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "paged decode is built for bf16 only");
  const size_t need = ws_bytes(B, H, d, S);
  fa_status st = check_workspace(workspace, workspace_bytes, need);
  if (st != FA_OK) return st;
  const Range rw = span(workspace, need);
  if (overlap(rw, rq) || overlap(rw, rk) || overlap(rw, rv) || overlap(rw, rt) || overlap(rw, rs) ||
      overlap(rw, ro) || (lse && overlap(rw, rl)))
    return fail(FA_ERR_INVALID_ARG, "workspace overlaps another tensor");
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o + (size_t)B * H * S * d;
  const fa_status pend = take_pending("fa_decode_paged");
  if (pend != FA_OK) return pend;
  if (mfma_path) {
    // the G query heads of a key/value head are the query rows of one split forward over its pages
    fa::PrefillArgs a{q, k_pages, v_pages, nullptr, nullptr, B, H_kv, G, (int)max_len, d, scale, false};
    a.splits = S;
    a.ws_o = ws_o;
    a.ws_lse = ws_lse;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.num_pages = num_pages;
    a.page_size = page_size;
    a.max_blocks = max_blocks;
    st = device_status(fa::launch_prefill_paged_bf16(a, (hipStream_t)stream), "fa_decode_paged split launch");
  } else {
    fa::PagedDecodeArgs a{q, k_pages, v_pages, block_table, seq_lens, B, H, H_kv, num_pages, page_size, max_blocks,
                          d, scale, S, ws_o, ws_lse};
    st = device_status(fa::launch_decode_paged_bf16(a, (hipStream_t)stream), "fa_decode_paged split launch");
  }
  if (st != FA_OK) return st;
  fa::CombineArgs cmb{ws_o, ws_lse, o, lse, B, H, d, S};
  return device_status(fa::launch_decode_combine_bf16(cmb, (hipStream_t)stream), "fa_decode_paged combine launch");
}

size_t fa_bwd_workspace_bytes(int B, int H, int N_q) {
  int64_t n;
  if (B < 1 || H < 1 || N_q < 1 || !mul_ok(n, {B, H, N_q, 4}) || n > kMaxElems) return 0;
  return (size_t)n;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, int B, int H, int N_q, int N_kv, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream, fa_dtype dtype) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARG, "q, k, v, o, lse, dout, dq, dk and dv must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
    return fail(FA_ERR_INVALID_ARG, "tensors must be 16-byte aligned (lse 4-byte)");
  if (B < 1 || H < 1 || N_q < 1 || N_kv < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H, N_q, N_kv must be >= 1 (got %d, %d, %d, %d)", B, H, N_q, N_kv);
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head size d=%d is not built (supported: 64, 128)", d);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  if (causal && N_q > N_kv)
    return fail(FA_ERR_INVALID_ARG, "causal attention needs N_q <= N_kv (got N_q=%d, N_kv=%d)", N_q, N_kv);
  if (dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "the backward is built for bf16 only");
  int64_t nq_el, nkv_el;
  if (!mul_ok(nq_el, {B, H, N_q, d}) || !mul_ok(nkv_el, {B, H, N_kv, d}) || nq_el > kMaxElems || nkv_el > kMaxElems)
    return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  if ((int64_t)N_kv * d * 2 > INT_MAX || (int64_t)N_q * d * 2 > INT_MAX)
    return fail(FA_ERR_UNSUPPORTED, "the backward supports N * d * 2 <= 2^31 - 1 bytes per head");
  if (fa::bwd_bf16_grid(B, H, N_q, N_kv) > INT_MAX) return fail(FA_ERR_INVALID_ARG, "launch grid too large");
  const size_t need = fa_bwd_workspace_bytes(B, H, N_q);
  fa_status st = check_workspace(workspace, workspace_bytes, need);
  if (st != FA_OK) return st;
  const Range rq = span(q, nq_el * 2), rk = span(k, nkv_el * 2), rv = span(v, nkv_el * 2), ro = span(o, nq_el * 2),
              rdo = span(dout, nq_el * 2), rl = span(lse, (size_t)B * H * N_q * 4), rw = span(workspace, need);
  const Range outs[4] = {span(dq, nq_el * 2), span(dk, nkv_el * 2), span(dv, nkv_el * 2), rw};
  const Range ins[6] = {rq, rk, rv, ro, rdo, rl};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], ins[j])) return fail(FA_ERR_INVALID_ARG, "an output or the workspace overlaps an input");
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(FA_ERR_INVALID_ARG, "outputs / workspace overlap each other");
  }
  fa::BwdArgs a{q, k, v, o, dout, lse, static_cast<float*>(workspace), dq, dk, dv, B, H, N_q, N_kv, d, scale,
                causal != 0};
  a.num_cu = fa::planning_cu_count();
  const fa_status pend = take_pending("fa_bwd");
  if (pend != FA_OK) return pend;
  return device_status(fa::launch_bwd_bf16(a, (hipStream_t)stream), "fa_bwd launch");
}

int fa_device_num_cu(void) { return fa::device_cu_count(); }

fa_status fa_plan(fa_plan_op op, int B, int H, int N_q, int N_kv, int d, int causal, fa_dtype dtype, int num_splits,
                  int num_cu, fa_plan_info* out) {
  if (!out) return fail(FA_ERR_INVALID_ARG, "out must be non-NULL");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 1 || H < 1 || N_q < 1 || N_kv < 1 || num_cu < 0 || num_splits < 0)
    return fail(FA_ERR_INVALID_ARG, "B, H, N_q, N_kv must be >= 1 and num_cu, num_splits >= 0");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head size d=%d is not built (supported: 64, 128)", d);
  if (op != FA_PLAN_FWD && dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "only fa_fwd is built for fp32");
  const int cu = num_cu > 0 ? num_cu : fa::planning_cu_count();
  fa::LaunchPlan pl;
  int S = 0;
  switch (op) {
    case FA_PLAN_FWD:
      pl = dtype == FA_DTYPE_BF16 ? fa::plan_prefill_bf16(B, H, N_q, d, causal != 0, 0, cu)
                                  : fa::plan_prefill_f32(B, H, N_q, d, cu);
      break;
    case FA_PLAN_FWD_SPLIT:
      S = num_splits > 0 ? num_splits : fwd_split_auto(B, H, N_q, N_kv, cu);
      pl = fa::plan_prefill_bf16(B, H, N_q, d, causal != 0, S, cu);
      break;
    case FA_PLAN_DECODE:
      S = num_splits > 0 ? num_splits : auto_splits(B, H, N_kv, cu);
      pl.kernel = fa::kKernelDecodeSplit;
      pl.waves = 8;
      pl.rows = 1;
      pl.groups = (int64_t)B * H * S;
      break;
    case FA_PLAN_BWD_DQ:
      pl = fa::plan_bwd_dq(B, H, N_q, d, causal != 0, cu);
      break;
    case FA_PLAN_BWD_DKDV:
      pl = fa::plan_bwd_dkdv(B, H, N_kv, d, causal != 0, cu);
      break;
    default:
      return fail(FA_ERR_INVALID_ARG, "unknown plan op %d", (int)op);
  }
  out->kernel = pl.kernel;
  out->waves_per_group = pl.waves;
  out->rows_per_group = pl.rows;
  out->paired = pl.paired ? 1 : 0;
  out->groups = pl.groups;
  out->num_splits = S;
  return FA_OK;
}

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_DEVICE: return "FA_ERR_DEVICE";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_err; }

const char* fa_version(void) { return "libfa 0.1 gfx950"; }

}  // extern "C"
