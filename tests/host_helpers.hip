// Test shim: the GPU path's number-format and exp helpers compiled for the
// host, so that their logic can be compared with the oracle on the CPU before
// any GPU run. The GPU tests check the same helpers as compiled for gfx950.
#include <stdint.h>
#include "../long_context_sparse_indexer_amd/csrc/device.hpp"

extern "C" {
void ht_e4m3_from_bf16(const uint16_t* in, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)s5::e4m3_from_bf16(in[i]);
}
void ht_bf16_bits(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)s5::bf16_bits(in[i]);
}
void ht_exp(const float* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = s5::exp_fixed(in[i]);
}
float ht_pair8(const float* a) { return s5::pair8(a); }
}
