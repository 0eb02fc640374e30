// Instantiation and choice of the forward kernels for FP8 E4M3 inputs.  A translation unit of
// its own, so that the library build compiles it alongside fa_api.hip.
#include <hip/hip_runtime.h>

#include "fa_fwd_bf16_pipe.h"
#include "fa_fwd_ksplit.h"

namespace fa {
namespace {

template <int D, bool CAUSAL, bool PAD, bool OUTF32>
FwdKernelFn fp8_nw(bool wide, bool small, int* bm, int* threads) {
    if (small) {   // key split: eight waves at d = 64, four at d = 128
        constexpr int NW = D == 64 ? 8 : 4;
        *bm = 32;
        *threads = 64 * NW;
        return fa_fwd_bf16_ksplit_kernel<D, CAUSAL, PAD, OUTF32, NW, true>;
    }
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
FwdKernelFn fp8_mask(int mask, bool wide, bool small, int* bm, int* threads) {
    switch (mask) {
        case 0: return fp8_nw<D, false, false, OUTF32>(wide, small, bm, threads);
        case 1: return fp8_nw<D, true, false, OUTF32>(wide, small, bm, threads);
        case 2: return fp8_nw<D, false, true, OUTF32>(wide, small, bm, threads);
        default: return fp8_nw<D, true, true, OUTF32>(wide, small, bm, threads);
    }
}

}  // namespace

FwdKernelFn pick_fp8_kernel(int d, int mask, bool out_f32, bool wide, bool small, int* bm, int* threads) {
    if (d == 64)
        return out_f32 ? fp8_mask<64, true>(mask, false, small, bm, threads) : fp8_mask<64, false>(mask, false, small, bm, threads);
    if (d == 128)
        return out_f32 ? fp8_mask<128, true>(mask, wide, small, bm, threads) : fp8_mask<128, false>(mask, wide, small, bm, threads);
    return nullptr;
}

}  // namespace fa
