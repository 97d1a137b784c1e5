// Host build of the library's device codec (fp8_moe_ffn_amd/csrc/codec.hpp), so a
// CPU test can compare the exact source the kernels use with the oracle.
#include "codec.hpp"

extern "C" {
void host_encode(const float* v, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)moe::e4m3_encode(v[i], 0);
}
void host_encode_div(const float* v, const float* s, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)moe::e4m3_encode_div(v[i], s[i]);
}
void host_decode(const uint8_t* c, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = moe::e4m3_decode(c[i]);
}
void host_bf16(const float* v, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = moe::float_to_bf16(v[i]);
}
}
