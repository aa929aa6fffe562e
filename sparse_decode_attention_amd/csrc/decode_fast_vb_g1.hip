// Matrix-core decode over a cache whose V is pruned in 8-channel blocks, for
// G = 1 query heads per KV head: the runtime-T variants (row lengths up to
// 32, 64, 96 and 128, even and odd).
#include "decode_fast.h"

namespace spark {

hipError_t launch_fast_vb_g1(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    return launch_fast_rt_v<1, true>(a, grid, stream);
}

}  // namespace spark
