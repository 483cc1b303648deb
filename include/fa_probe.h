/*
 * fa_probe.h -- measurement probes exported by libfa next to the attention entry points of fa.h.
 *
 * They measure the machine, not the method: the read bandwidth a plain streaming kernel reaches from
 * HBM, and the shader clock the chip holds under dense matrix-core load.  Benchmarks report them beside
 * the attention kernels' figures, so that a memory-bound kernel can be read against what a plain read
 * achieves and a matrix-core-bound one against the clock actually running (context for the throughput
 * comparisons of "FlashAttention Explained: How AI Models Process Attention Faster and Use Less
 * Memory", section "How to Benchmark Performance").  Return codes: 0 = launched, 1 = invalid argument
 * (nothing launched), 4 = the HIP runtime refused the launch or an error from earlier work was pending
 * (nothing launched in that case).  Work is enqueued on `stream` (a hipStream_t, NULL = null stream).
 */
#ifndef FA_PROBE_H_
#define FA_PROBE_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads the first bytes / 16 * 16 bytes at buf (device memory, 16-byte aligned, bytes >= 16) once with
 * 16-byte non-temporal loads.  Each of `groups` work-groups of 512 threads streams one contiguous
 * span of about bytes / groups bytes, four coalesced 8 KB loads in flight per step (two groups per
 * compute unit read fastest).  Each thread stores a fold of what it read into sink (device memory,
 * 4-byte aligned, sink_bytes >= groups * 512 * 4), so the loads cannot be optimised away.
 * Bandwidth = bytes / (the kernel's duration).
 */
int fa_probe_read_bandwidth(const void* buf, size_t bytes, void* sink, size_t sink_bytes, int groups, void* stream);

/*
 * Runs `groups` work-groups of 256 threads, each issuing ceil(iters / 8) x 64 bf16 32x32x16 MFMAs per wave on
 * pseudo-random operands that change every instruction.  Work-group g writes out[5g .. 5g+4] (device
 * memory, 8-byte aligned, out_words >= 5 * groups): the shader clock counter (s_memtime) and the
 * 100 MHz constant counter (s_memrealtime) before the loop, the same two after it, and a flag that
 * is 0 unless the accumulators became NaN.  The clock in MHz over the loop is
 * 100 * (t1 - t0) / (r1 - r0).
 */
int fa_probe_clock(unsigned long long* out, size_t out_words, int groups, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */
