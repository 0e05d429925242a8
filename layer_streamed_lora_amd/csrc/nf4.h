// NF4 code table passed to kernels by value (kernel arguments live in the
// constant kernarg segment, so no device-global state is needed).
#pragma once
namespace lsl {
struct Nf4Table {
  float cb[16];   // code values, ascending
  float mid[16];  // mid[i] = (cb[i] + cb[i+1]) / 2 in float32, i < 15
};
const Nf4Table& nf4_table();
void nf4_codebook_host(float out[16]);
}  // namespace lsl
