// Instantiation and choice of the forward kernels for FP8 E4M3 inputs.  A translation unit of
// its own, so that the library build compiles it alongside fa_api.hip.
#include <hip/hip_runtime.h>

#include "fa_fwd_bf16_pipe.h"

namespace fa {
namespace {

template <int D, bool CAUSAL, bool PAD, bool OUTF32>
FwdKernelFn fp8_nw(bool wide, int* bm, int* threads) {
    if constexpr (D == 128 && CAUSAL) {
        if (wide) {   // one eight-wave, 256-row workgroup per CU (long causal d = 128 heads)
            *bm = 256;
            *threads = 512;
            return fa_fwd_fp8_pipe_kernel<D, 64, CAUSAL, PAD, OUTF32, 8>;
        }
    }
    *bm = 128;
    *threads = 256;
    return fa_fwd_fp8_pipe_kernel<D, 64, CAUSAL, PAD, OUTF32, 4>;
}

template <int D, bool OUTF32>
FwdKernelFn fp8_mask(int mask, bool wide, int* bm, int* threads) {
    switch (mask) {
        case 0: return fp8_nw<D, false, false, OUTF32>(wide, bm, threads);
        case 1: return fp8_nw<D, true, false, OUTF32>(wide, bm, threads);
        case 2: return fp8_nw<D, false, true, OUTF32>(wide, bm, threads);
        default: return fp8_nw<D, true, true, OUTF32>(wide, bm, threads);
    }
}

}  // namespace

FwdKernelFn pick_fp8_kernel(int d, int mask, bool out_f32, bool wide, int* bm, int* threads) {
    if (d == 64) return out_f32 ? fp8_mask<64, true>(mask, false, bm, threads) : fp8_mask<64, false>(mask, false, bm, threads);
    if (d == 128) return out_f32 ? fp8_mask<128, true>(mask, wide, bm, threads) : fp8_mask<128, false>(mask, wide, bm, threads);
    return nullptr;
}

}  // namespace fa
