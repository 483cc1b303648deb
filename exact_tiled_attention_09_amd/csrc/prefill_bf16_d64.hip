// The d = 64 instances of the bf16 prefill kernel (prefill_bf16.hip) in a compilation unit of their own,
// so that they can be built with the LLVM scheduler strategy that measured fastest for them (iterative
// ILP, see build.py); the d = 128 instances keep the default strategy, which is faster for them.
#define FA_PREFILL_D64_UNIT 1
#include "prefill_bf16.hip"
