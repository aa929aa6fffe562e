// Matrix-core decode for G = 1 query heads per KV head: the runtime-T
// variants (row lengths up to 32, 64, 96 and 128, even and odd) and the
// ragged-row variant.
#include "decode_fast.h"

namespace spark {

hipError_t launch_fast_g1(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    return launch_fast_rt<1>(a, grid, stream);
}

}  // namespace spark
