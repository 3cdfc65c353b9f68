// bfloat16-cache instantiations of the decode kernel.
#include "pa_decode_kernel.h"

namespace pa {
bool launch_decode_bf16(int d, int bs, int g, const DecodeArgs& a, dim3 grid, int waves,
                        size_t lds, hipStream_t s) {
  return launch_decode_impl<kBF16>(d, bs, g, a, grid, waves, lds, s);
}
int decode_groups_per_cu_bf16(int d, int bs, int g, int waves, size_t lds) {
  return decode_groups_per_cu_impl<kBF16>(d, bs, g, waves, lds);
}
}  // namespace pa
