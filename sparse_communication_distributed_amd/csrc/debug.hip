// Debug check of the inputs: a count of non-finite values (NaN, +-inf) in
// an fp32 array.  The step itself computes on whatever it is given (a NaN
// key sorts above +inf in the selection, and NaN or inf propagate through
// the compression and AdamS as IEEE 754 arithmetic does); this count lets a
// caller see such inputs without reading the array back.

#include "scape_internal.h"

namespace scape {
namespace {

__device__ __forceinline__ uint32_t nonfinite(float x) {
  return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u ? 1u : 0u;
}

// Grid-stride count over x[0 .. n-1]; VEC: x 16-byte aligned, 4 elements a
// load for the first n - n % 4.  One atomic per wave that saw any.
template <bool VEC>
__global__ void __launch_bounds__(kThreads)
nonfinite_kernel(const float* __restrict__ x, int64_t n, unsigned long long* __restrict__ out) {
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t nth = (int64_t)gridDim.x * kThreads;
  uint32_t c = 0;
  int64_t head = 0;
  if (VEC) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    const int64_t n4 = n / 4;
    const v4f* x4 = reinterpret_cast<const v4f*>(x);
    for (int64_t i = tid; i < n4; i += nth) {
      const v4f v = __builtin_nontemporal_load(x4 + i);
      c += nonfinite(v.x) + nonfinite(v.y) + nonfinite(v.z) + nonfinite(v.w);
    }
    head = n4 * 4;
  }
  for (int64_t i = head + tid; i < n; i += nth) c += nonfinite(x[i]);
  uint64_t s = c;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  if ((threadIdx.x & 63) == 0 && s) atomicAdd(out, (unsigned long long)s);
}

}  // namespace

hipError_t launch_count_nonfinite(const float* x, int64_t n, uint64_t* out, hipStream_t s) {
  if (n < 1) return hipSuccess;
  int64_t blocks = (n / 4 + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  unsigned long long* o = reinterpret_cast<unsigned long long*>(out);
  if ((reinterpret_cast<uintptr_t>(x) & 15u) == 0)
    nonfinite_kernel<true><<<(unsigned)blocks, kThreads, 0, s>>>(x, n, o);
  else
    nonfinite_kernel<false><<<(unsigned)blocks, kThreads, 0, s>>>(x, n, o);
  return hipGetLastError();
}

}  // namespace scape
