// Matrix-core decode, exact-T variants: G = 4 query heads per KV head and the
// row lengths of the pruning ratios in common use (T = 26, 38, 48, 64: lambda
// 0.8, 0.7, 0.625, 0.5 at D = 128), with the fixed or sampled recovery F.
#include "decode_fast.h"

namespace spark {

namespace {

template <int SMODE>
hipError_t launch_fixed_smode(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    switch (a.T) {
        case 26: return launch_fast_variant<4, 26, 26, false, SMODE, false>(a, grid, stream);
        case 38: return launch_fast_variant<4, 38, 38, false, SMODE, false>(a, grid, stream);
        case 48: return launch_fast_variant<4, 48, 48, false, SMODE, false>(a, grid, stream);
        case 64: return launch_fast_variant<4, 64, 64, false, SMODE, false>(a, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fast_fixed(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    switch (a.sampled) {
        case 0: return launch_fixed_smode<0>(a, grid, stream);
        case 4: return launch_fixed_smode<4>(a, grid, stream);
        case 5: return launch_fixed_smode<5>(a, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spark
