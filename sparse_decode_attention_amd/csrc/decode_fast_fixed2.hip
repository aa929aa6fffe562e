// Matrix-core decode, more exact-T variants with the fixed recovery F: G = 4
// at the other pruning ratios of a lambda sweep in steps of 0.1 (T = 13, 51,
// 77, 90, 102, 115: lambda 0.9, 0.6, 0.4, 0.3, 0.2, 0.1 at D = 128), and
// G = 1, 2, 8 at lambda 0.8 and 0.5 (T = 26, 64).
#include "decode_fast.h"

namespace spark {

namespace {

template <int T>
hipError_t launch_exact(const DecodeArgs& a, int G, dim3 grid, hipStream_t stream) {
    switch (G) {
        case 1: return launch_fast_variant<1, T, T, (T & 1) != 0, 0, false>(a, grid, stream);
        case 2: return launch_fast_variant<2, T, T, (T & 1) != 0, 0, false>(a, grid, stream);
        case 8: return launch_fast_variant<8, T, T, (T & 1) != 0, 0, false>(a, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fast_fixed2(const DecodeArgs& a, int G, dim3 grid, hipStream_t stream) {
    if (a.sampled) return hipErrorInvalidValue;
    if (G == 4) {
        switch (a.T) {
            case 13: return launch_fast_variant<4, 13, 13, true, 0, false>(a, grid, stream);
            case 51: return launch_fast_variant<4, 51, 51, true, 0, false>(a, grid, stream);
            case 77: return launch_fast_variant<4, 77, 77, true, 0, false>(a, grid, stream);
            case 90: return launch_fast_variant<4, 90, 90, false, 0, false>(a, grid, stream);
            case 102: return launch_fast_variant<4, 102, 102, false, 0, false>(a, grid, stream);
            case 115: return launch_fast_variant<4, 115, 115, true, 0, false>(a, grid, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.T) {
        case 26: return launch_exact<26>(a, G, grid, stream);
        case 64: return launch_exact<64>(a, G, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spark
