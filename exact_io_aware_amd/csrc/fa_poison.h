// LDS poisoning for the test build (libfa_poison.so, compiled with
// FA_POISON_LDS=1): each kernel fills its LDS data buffers with all-ones
// bytes (NaN as fp32, bf16 and fp16) and waits at a barrier before its
// first use.  A read of LDS that none of the kernel's own loads or stores
// wrote then turns the results it feeds into NaN, where the normal build
// would silently reuse whatever the buffer held.  Index arrays (the sparse
// tile list) are not poisoned: a garbage index could address out of bounds.
// In the normal build every call compiles to nothing.
#ifndef FA_POISON_H
#define FA_POISON_H

#include <hip/hip_runtime.h>

#include <cstdint>

#ifndef FA_POISON_LDS
#define FA_POISON_LDS 0
#endif

namespace fa {

// Fill `bytes` (a multiple of 4) of LDS at p, all threads of the block
// taking part; the caller ends the fills with one __syncthreads().
__device__ __forceinline__ void poison_lds(void* p, int bytes, int tid, int nthreads) {
  if constexpr (FA_POISON_LDS != 0) {
    uint32_t* w = (uint32_t*)p;
    for (int i = tid; i < bytes / 4; i += nthreads) w[i] = 0xffffffffu;
  }
}

constexpr bool kPoisonLds = FA_POISON_LDS != 0;

}  // namespace fa

#endif  // FA_POISON_H
