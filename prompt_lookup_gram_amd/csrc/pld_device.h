// Device helpers shared by the context-store kernels (the n-gram index and
// the successor-count cache): a token-sequence hash and the view of a
// request's history while an append is in flight.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pld {

// Hash of a token sequence, one step per token, then a final mix. The step
// multiplies by the 64-bit golden-ratio constant (2^64 / phi, Fibonacci
// hashing as in Knuth's multiplicative method); the final mix is the fmix64
// finaliser of Austin Appleby's MurmurHash3 (its published shift and
// multiplier constants). The seed is the first 64 bits of pi's fraction.
// Hash quality only affects speed: every hit is confirmed on the tokens.
__device__ __forceinline__ unsigned long long hstep(unsigned long long h, int32_t t)
{
    h ^= (uint32_t)t;
    h *= 0x9e3779b97f4a7c15ull;
    return h ^ (h >> 29);
}

__device__ __forceinline__ unsigned long long hfinal(unsigned long long h)
{
    h ^= h >> 33;
    h *= 0xff51afd7ed558ccdull;
    h ^= h >> 33;
    h *= 0xc4ceb9fe1a85ec53ull;
    return h ^ (h >> 33);
}

constexpr unsigned long long kHashSeed = 0x243f6a8885a308d3ull;

// Token q of request b during an append: from the store below the old
// length, from the append's source row above it.
struct AppendView {
    const int32_t *store_row;
    const int32_t *src;
    int32_t old_len;
    __device__ __forceinline__ int32_t at(int64_t q) const
    {
        // one load from whichever buffer holds q
        const int32_t *p = q < old_len ? store_row + q : src + (q - old_len);
        return *p;
    }
};

}  // namespace pld
