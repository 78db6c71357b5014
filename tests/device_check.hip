// GPU checks of the hardware conversions the kernels use against the software
// forms (bf16_bits, e4m3_from_bf16), which the CPU tests pin to the oracle.
// Built by __graft_entry__.build() into tests/_device_check.so; each entry
// point takes device pointers and launches one kernel on the null stream.
#include "../long_context_sparse_indexer_amd/csrc/device.hpp"

using namespace s5;

// every fp32 bit pattern except NaNs: bf16x2_hw(x, -x) against bf16_bits
__global__ void check_bf16_kernel(unsigned long long* mismatches, uint32_t* first) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  unsigned long long bad = 0;
  for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < (1ull << 32); u += stride) {
    const uint32_t w = (uint32_t)u;
    if ((w & 0x7fffffffu) > 0x7f800000u) continue;  // NaN
    const float x = __builtin_bit_cast(float, w);
    const uint32_t hw = bf16x2_hw(x, -x);
    const uint32_t sw = bf16_bits(x) | (bf16_bits(-x) << 16);
    if (hw != sw) {
      ++bad;
      atomicMin(first, w);
    }
  }
  if (bad) atomicAdd(mismatches, bad);
}

// every bf16 bit pattern except NaNs and infinities: e4m3x2_hw against
// e4m3_from_bf16, both halves of the register and both word positions
__global__ void check_e4m3_kernel(unsigned long long* mismatches, uint32_t* first) {
  const uint32_t h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= 65536u) return;
  if ((h & 0x7f80u) == 0x7f80u) return;  // Inf / NaN
  const uint32_t h2 = h ^ 0x8000u;
  const float a = __builtin_bit_cast(float, h << 16), b = __builtin_bit_cast(float, h2 << 16);
  const uint32_t sw = e4m3_from_bf16(h) | (e4m3_from_bf16(h2) << 8);
  const uint32_t lo = e4m3x2_hw<false>(a, b, 0u);
  const uint32_t hi = e4m3x2_hw<true>(a, b, 0x5a5au);
  if ((lo & 0xffffu) != sw || (hi >> 16) != sw || (hi & 0xffffu) != 0x5a5au) {
    atomicAdd(mismatches, 1ull);
    atomicMin(first, h);
  }
}

extern "C" __attribute__((visibility("default"))) int device_check_bf16(unsigned long long* mismatches, uint32_t* first) {
  hipLaunchKernelGGL(check_bf16_kernel, dim3(4096), dim3(256), 0, 0, mismatches, first);
  return (int)hipDeviceSynchronize();
}
extern "C" __attribute__((visibility("default"))) int device_check_e4m3(unsigned long long* mismatches, uint32_t* first) {
  hipLaunchKernelGGL(check_e4m3_kernel, dim3(256), dim3(256), 0, 0, mismatches, first);
  return (int)hipDeviceSynchronize();
}

// exp_fixed (the summary's exp) on the inputs whose fp32 bit patterns are
// start, start + 1, ..., start + n - 1 (out[i] for start + i)
__global__ void exp_range_kernel(uint32_t start, uint32_t n, float* out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = exp_fixed(__builtin_bit_cast(float, start + i));
}
// exp_fixed of n given inputs
__global__ void exp_list_kernel(const float* in, float* out, uint32_t n) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = exp_fixed(in[i]);
}

extern "C" __attribute__((visibility("default"))) int device_exp_range(uint32_t start, uint32_t n,
                                                                       float* out) {
  if (n == 0 || n > (1u << 30)) return -1;
  hipLaunchKernelGGL(exp_range_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, start, n, out);
  return (int)hipDeviceSynchronize();
}
extern "C" __attribute__((visibility("default"))) int device_exp_list(const float* in, float* out,
                                                                      uint32_t n) {
  if (n == 0 || n > (1u << 30)) return -1;
  hipLaunchKernelGGL(exp_list_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, in, out, n);
  return (int)hipDeviceSynchronize();
}
