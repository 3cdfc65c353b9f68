// 8-bit (E4M3)-cache instantiations of the prefill attention kernel.
#include "pa_prefill_kernel.h"

namespace pa {
namespace pf {
int launch_prefill_fp8(const PrefillArgs& a, int block_size, int group, bool out_f32,
                        dim3 grid, hipStream_t stream) {
  return launch_et<kFP8>(a, block_size, group, out_f32, grid, stream);
}
}  // namespace pf
}  // namespace pa
