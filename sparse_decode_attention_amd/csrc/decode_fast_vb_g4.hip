// Matrix-core decode over a cache whose V is pruned in 8-channel blocks, for
// G = 4 query heads per KV head: the runtime-T variants (row lengths up to
// 32, 64, 96 and 128, even and odd) and the exact-T variants of lambda 0.5 and
// 0.8 (T = 64, 26).
#include "decode_fast.h"

namespace spark {

hipError_t launch_fast_vb_g4(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    if (a.T == 64) return launch_fast_variant<4, 64, 64, false, 0, false, true>(a, grid, stream);
    if (a.T == 26) return launch_fast_variant<4, 26, 26, false, 0, false, true>(a, grid, stream);
    return launch_fast_rt_v<4, true>(a, grid, stream);
}

}  // namespace spark
