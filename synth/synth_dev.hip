// Device implementation of the normal stream defined in synth.h, used to fill
// large weight tensors directly in HBM.  Same definition as synth.c; a GPU test
// checks the two agree bit for bit on sampled elements.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t at(uint64_t key, uint64_t i) {
  return mix(key + (i + 1u) * 0x9E3779B97F4A7C15ull);
}
__device__ __forceinline__ double unif(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }

__global__ void fill_normal_bf16(uint64_t key, double std, uint64_t first, uint64_t n, uint16_t* out) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    const uint64_t e = first + i;
    double u1 = unif(at(key, 2u * e));
    double u2 = unif(at(key, 2u * e + 1u));
    double z = sqrt(-2.0 * log(1.0 - u1)) * cos(two_pi * u2);
    float f = (float)(std * z);
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    out[i] = (uint16_t)(b >> 16);
  }
}

}  // namespace

extern "C" int synth_dev_normal_bf16(uint64_t seed, uint64_t stream, double std, uint64_t first, uint64_t n,
                                     void* d_out, void* stream_handle) {
  if (n == 0) return 0;
  if (d_out == nullptr) return -1;
  // key(seed, stream) = at(seed, stream), computed on the host side of this call.
  uint64_t z = seed + (stream + 1u) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  const uint64_t key = z ^ (z >> 31);
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_normal_bf16, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream_handle, key, std, first,
                     n, (uint16_t*)d_out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
