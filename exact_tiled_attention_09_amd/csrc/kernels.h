// Host-side launchers of the gfx950 attention kernels (internal to libfa; the C ABI lives in fa_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Compute units of the full MI355X / MI350X (8 XCDs x 32): the launch heuristics' assumption when the
// device cannot be asked (host-only sizing calls on a machine without a visible device).
constexpr int kDefaultNumCu = 256;

// Compute units of the current device, read once per device and cached; 0 if no device can be queried.
int device_cu_count();
// device_cu_count(), or kDefaultNumCu when it is 0.
int planning_cu_count();

// Kernel identifiers reported by fa_plan (values of fa_kernel_id in fa.h).
enum KernelId : int {
  kKernelBf16FourWave = 1,
  kKernelBf16EightWave = 2,
  kKernelBf16Split = 3,
  kKernelF32Rows = 4,
  kKernelF32KeySplit = 5,
  kKernelDecodeSplit = 6,
  kKernelBwdDq = 7,
  kKernelBwdDkdv = 8,
};

// A launch decision: which kernel, its work-group shape and grid.
struct LaunchPlan {
  int kernel = 0;
  int waves = 0;          // waves per work-group
  int rows = 0;           // query rows (keys for the dK/dV kernel) per work-group
  bool paired = false;    // causal tiles n-1-j and j in one work-group
  int64_t groups = 0;     // work-groups launched
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Nq, Nkv, d;
  float scale;
  bool causal;
  // split-KV forward (bf16): splits > 0 writes per-range partials instead of o / lse
  int splits = 0;
  float* ws_o = nullptr;    // [B*H*N_q, splits, d]
  float* ws_lse = nullptr;  // [B*H*N_q, splits]
  // paged key/value cache (launch_prefill_paged_bf16 only): H counts key/value heads, k and v are page pools
  // [num_pages, H, page_size, d], N_kv is unused (lengths come from seq_lens on the device)
  const int* block_table = nullptr;  // [B, max_blocks]
  const int* seq_lens = nullptr;     // [B]
  int num_pages = 0, page_size = 0, max_blocks = 0;
  int num_cu = kDefaultNumCu;  // compute units of the device the launch goes to (sizes pairing and wave counts)
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  int B, H, Nkv, d;
  float scale;
  int splits;
  float* ws_o;    // [B,H,S,d]
  float* ws_lse;  // [B,H,S]
};

struct PagedDecodeArgs {
  const void* q;        // [B, H, d]
  const void* k_pages;  // [num_pages, H_kv, page_size, d]
  const void* v_pages;
  const int* block_table;  // [B, max_blocks]
  const int* seq_lens;     // [B]
  int B, H, Hkv, num_pages, page_size, max_blocks, d;
  float scale;
  int splits;
  float* ws_o;    // [B*H, S, d]
  float* ws_lse;  // [B*H, S]
};

struct CombineArgs {
  const float* ws_o;
  const float* ws_lse;
  void* o;
  float* lse;
  int B, H, d, splits;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;  // workspace [B,H,N_q]
  void* dq;
  void* dk;
  void* dv;
  int B, H, Nq, Nkv, d;
  float scale;
  bool causal;
  int num_cu = kDefaultNumCu;
};

// Each launcher assumes validated arguments and returns the launch status.
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
// Split mode over a paged cache, no mask: writes the split partials of N_q query rows per key/value head.
// Needs page_size >= 8 (a 1 KB load block never straddles a page).
hipError_t launch_prefill_paged_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode_split_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_combine_bf16(const CombineArgs& a, hipStream_t s);
hipError_t launch_decode_paged_bf16(const PagedDecodeArgs& a, hipStream_t s);  // G = H / H_kv in {1, 2, 4, 8}
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);

// The launch decisions of the launchers above, for a device with num_cu compute units.
LaunchPlan plan_prefill_bf16(int B, int H, int Nq, int d, bool causal, int splits, int num_cu);
LaunchPlan plan_prefill_f32(int B, int H, int Nq, int d, int num_cu);
LaunchPlan plan_bwd_dq(int B, int H, int Nq, int d, bool causal, int num_cu);
LaunchPlan plan_bwd_dkdv(int B, int H, int Nkv, int d, bool causal, int num_cu);

// Grid-size helpers shared with argument validation.
int64_t prefill_bf16_grid(int B, int H, int Nq, int d, int splits = 0);
int prefill_split_tiles(int Nkv, int S);  // 64-key tiles per split of the split-KV forward
int64_t prefill_f32_grid(int B, int H, int Nq, int d);
int64_t bwd_bf16_grid(int B, int H, int Nq, int Nkv);

}  // namespace fa
