// C ABI of the fused attention forward (declared in include/fa.h): host-side validation,
// kernel selection and launch.  No allocation and no synchronisation.  State: the thread-local
// last HIP error, and for fa_fwd_varlen_noalloc a fixed device array with its per-device address.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/fa.h"
#include "fa_fwd_bf16.h"
#include "fa_fwd_bf16_pipe.h"
#include "fa_fwd_f32.h"
#include "fa_fwd_ksplit.h"
#include "fa_bwd_bf16.h"
#include "fa_decode_bf16.h"

// Workspace of fa_fwd_varlen_noalloc: the partial states of the split-key decoding kernel.  The
// largest plan needs bh * S * G * (d + 2) * 4 bytes with bh * S < 4096 (at most 2048 workgroups
// are aimed for, and a split needs fewer than 2048 (sequence, head) pairs), G <= 4 and d <= 128:
// 8,515,840 bytes, so 9 MiB holds every plan.  Each device the library runs on keeps its own
// copy until the process ends.
static __device__ __align__(256) unsigned char scratch[size_t{9} << 20];

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kScratchBytes = size_t{9} << 20;
static_assert(sizeof(scratch) == kScratchBytes, "one size for the array and its checks");
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device with that
// device current.  In host code the name `scratch` only stands for the symbol and must never
// reach a kernel: every use goes through the address returned here.
int scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = static_cast<int>(e);
        return FA_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            g_last_hip_error = static_cast<int>(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return FA_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

constexpr int kThreads = 256;  // 4 wave64s per workgroup

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

using Kernel = void (*)(fa::FwdArgs);

struct Launch {
    Kernel kern;
    int bm;            // query rows per tile
    bool paired;       // causal tiles are processed in pairs (one work item = tiles t and n-1-t)
    int threads = kThreads;
};

// Kernel variants, all computing the same function and passing the same tests:
//   0  software-pipelined kernel (direct-to-LDS loads, MFMA/VALU overlap)   -- production; the
//      eight-wave form of variant 3 for long causal d = 128 heads, else four waves
//   1  straightforward double-buffered kernel, LDS transpose reads of V
//   2  the same with V^T gathered by 16-bit LDS reads
//   3  the pipelined kernel with eight waves and 256-row tiles at every size (d = 128 only)
//   4  key split: the waves of a workgroup (8 at d = 64, 4 at d = 128) share 32 query rows and
//      divide the keys --
//      fa_fwd's choice when the grid of variant 0 would not fill the compute units
//   5  the four-wave pipelined kernel of variant 0 at every size (no automatic choice)
//   6  key split with 16-row query blocks (16x16x32 MFMAs; 8 waves at d = 64, 4 at d = 128) --
//      fa_fwd's choice for the smallest grids, where 32-row blocks leave compute units idle
constexpr int kNumVariants = 7;
// fa_fwd takes the key-split kernel when its own grid (one workgroup per 32 query rows) has at
// most this many workgroups -- at most two (d = 64, eight waves) or a half (d = 128, four
// waves) per compute unit of the 256 -- and there are at least this many keys per head.
// Measured on small grids against the four-wave pipelined kernel: inside these limits the key
// split was faster or level (0.98-2.1x), outside them slower (0.57-0.81x).  Below 512 keys a
// wave has at most one tile and splitting only adds the merge (N = 256: 0.68x).
constexpr int64_t kKeySplitMaxWgsD64 = 512;
constexpr int64_t kKeySplitMaxWgsD128 = 128;
constexpr int kKeySplitMinN = 512;
// ... and the 16-row key split (variant 6) when its grid, one workgroup per 16 query rows,
// fits one workgroup per compute unit.  Measured: N = 4096 single heads 15.2 vs 18.3 us
// (d = 64) and 35.4 vs 37.3 us (d = 128); with two 16-row workgroups per compute unit it was
// slower (N = 4096, two heads, d = 64: 25.0 vs 18.3 us).
constexpr int64_t kKeySplit16MaxWgs = 256;
// fa_fwd takes the eight-wave kernel for causal d = 128 launches with at least this many
// 256-row tiles (over all heads); smaller grids keep two 128-row workgroups per CU.
constexpr int64_t kWave8MinTiles = 1024;

template <int D, bool CAUSAL, bool PAD, bool OUTF32>
Launch pick_bf16_variant(int variant) {
    switch (variant) {
        case 0:
        case 5: return {fa::fa_fwd_bf16_pipe_kernel<D, 64, 1, CAUSAL, PAD, OUTF32>, 128, true};
        case 1: return {fa::fa_fwd_bf16_kernel<D, 64, CAUSAL, PAD, OUTF32, 1>, 128, false};
        case 2: return {fa::fa_fwd_bf16_kernel<D, 64, CAUSAL, PAD, OUTF32, 0>, 128, false};
        case 3:
            if constexpr (D == 128) return {fa::fa_fwd_bf16_pipe_kernel<D, 64, 1, CAUSAL, PAD, OUTF32, 8>, 256, true, 512};
            else return {nullptr, 0, false};
        case 4:   // eight waves at d = 64; four at d = 128, where eight would not fit the registers
            if constexpr (D == 64) return {fa::fa_fwd_bf16_ksplit_kernel<D, CAUSAL, PAD, OUTF32, 8>, 32, false, 512};
            else return {fa::fa_fwd_bf16_ksplit_kernel<D, CAUSAL, PAD, OUTF32, 4>, 32, false, 256};
        case 6:
            if constexpr (D == 64) return {fa::fa_fwd_bf16_ksplit16_kernel<D, CAUSAL, PAD, OUTF32, 8>, 16, false, 512};
            else return {fa::fa_fwd_bf16_ksplit16_kernel<D, CAUSAL, PAD, OUTF32, 4>, 16, false, 256};
        default: return {nullptr, 0, false};
    }
}

template <int D, bool OUTF32>
Launch pick_bf16_mask(int mask, int variant) {
    switch (mask) {
        case 0: return pick_bf16_variant<D, false, false, OUTF32>(variant);
        case 1: return pick_bf16_variant<D, true, false, OUTF32>(variant);
        case 2: return pick_bf16_variant<D, false, true, OUTF32>(variant);
        default: return pick_bf16_variant<D, true, true, OUTF32>(variant);
    }
}

template <int D>
Launch pick_f32_mask(int mask) {
    switch (mask) {
        case 0: return {fa::fa_fwd_f32_kernel<D, false, false>, 128, false};
        case 1: return {fa::fa_fwd_f32_kernel<D, true, false>, 128, false};
        case 2: return {fa::fa_fwd_f32_kernel<D, false, true>, 128, false};
        default: return {fa::fa_fwd_f32_kernel<D, true, true>, 128, false};
    }
}

// Dropout request of fa_fwd_dropout: drop probability, Philox seed and counter offset.
struct DropSpec {
    float p;
    uint64_t seed;
    uint32_t offset;
};

// Byte threshold round(256 p) of the dropout contract, or -1 when p is outside [0, 255.5/256).
int drop_threshold(float p) {
    if (!std::isfinite(p) || p < 0.f) return -1;
    const double t = std::floor(256.0 * static_cast<double>(p) + 0.5);
    return t <= 255.0 ? static_cast<int>(t) : -1;
}

template <int D, bool OUTF32>
Launch pick_bf16_drop(int mask) {
    switch (mask) {
        case 0: return {fa::fa_fwd_bf16_pipe_kernel<D, 64, 1, false, false, OUTF32, 4, true>, 128, true};
        case 1: return {fa::fa_fwd_bf16_pipe_kernel<D, 64, 1, true, false, OUTF32, 4, true>, 128, true};
        case 2: return {fa::fa_fwd_bf16_pipe_kernel<D, 64, 1, false, true, OUTF32, 4, true>, 128, true};
        default: return {fa::fa_fwd_bf16_pipe_kernel<D, 64, 1, true, true, OUTF32, 4, true>, 128, true};
    }
}

int launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int mask_kind, const int32_t* seqlens, int in_dtype, int out_dtype,
           void* stream, int variant, const DropSpec* drop = nullptr, const float* descale = nullptr) {
    // ---- validation (host only, before any HIP call) ----
    if (B < 0 || H < 0 || N < 0) return FA_ERR_INVALID_ARG;
    if (mask_kind < 0 || mask_kind > (FA_MASK_CAUSAL | FA_MASK_KEY_PADDING)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
    if (in_dtype != FA_DTYPE_F32 && in_dtype != FA_DTYPE_BF16 && in_dtype != FA_DTYPE_FP8_E4M3) return FA_ERR_INVALID_ARG;
    const bool f8 = in_dtype == FA_DTYPE_FP8_E4M3;
    // 8-bit inputs: per-tensor descales (Q, K, V); Q's and K's fold into the score multiplier
    const double dq = f8 && descale ? descale[0] : 1.0, dk = f8 && descale ? descale[1] : 1.0;
    const double dv = f8 && descale ? descale[2] : 1.0;
    if (!std::isfinite(dq) || !std::isfinite(dk) || !std::isfinite(dv) || dq < 0 || dk < 0 || dv < 0)
        return FA_ERR_INVALID_ARG;
    const double eff_scale = static_cast<double>(scale) * dq * dk;
    if (!std::isfinite(static_cast<float>(eff_scale)) || !std::isfinite(static_cast<float>(eff_scale * 1.4426950408889634074)))
        return FA_ERR_INVALID_ARG;
    if (out_dtype != FA_DTYPE_F32 && out_dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (d <= 0) return FA_ERR_INVALID_ARG;
    if (variant < 0 || variant >= kNumVariants) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (in_dtype == FA_DTYPE_F32 && out_dtype != FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
    if (in_dtype == FA_DTYPE_F32 && variant != 0) return FA_ERR_UNSUPPORTED;
    if (f8 && variant != 0) return FA_ERR_UNSUPPORTED;
    if (variant == 3 && d != 128) return FA_ERR_UNSUPPORTED;
    if (drop && drop_threshold(drop->p) < 0) return FA_ERR_INVALID_ARG;
    if (drop && in_dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
    if ((mask_kind & FA_MASK_KEY_PADDING) && !seqlens) return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
    if ((mask_kind & FA_MASK_KEY_PADDING) && !aligned(seqlens, 4)) return FA_ERR_INVALID_ARG;
    // ---- kernel selection ----
    // production choice: long causal d = 128 heads take the eight-wave kernel
    if (!drop && variant == 0 && in_dtype == FA_DTYPE_BF16 && d == 128 && (mask_kind & FA_MASK_CAUSAL) &&
        static_cast<int64_t>(B) * H * ((static_cast<int64_t>(N) + 255) / 256) >= kWave8MinTiles)
        variant = 3;
    // ... and grids too small to fill the chip take the key-split kernel
    if (!drop && variant == 0 && in_dtype == FA_DTYPE_BF16 && N >= kKeySplitMinN) {
        const int64_t wgs = static_cast<int64_t>(B) * H * ((static_cast<int64_t>(N) + 31) / 32);
        if (wgs <= (d == 64 ? kKeySplitMaxWgsD64 : kKeySplitMaxWgsD128)) variant = 4;
        if (variant == 4 && static_cast<int64_t>(B) * H * ((static_cast<int64_t>(N) + 15) / 16) <= kKeySplit16MaxWgs)
            variant = 6;
    }
    Launch L;
    if (drop) {
        const bool of32 = out_dtype == FA_DTYPE_F32;
        if (d == 64) L = of32 ? pick_bf16_drop<64, true>(mask_kind) : pick_bf16_drop<64, false>(mask_kind);
        else L = of32 ? pick_bf16_drop<128, true>(mask_kind) : pick_bf16_drop<128, false>(mask_kind);
    } else if (f8) {
        const bool wide = d == 128 && (mask_kind & FA_MASK_CAUSAL) &&
                          static_cast<int64_t>(B) * H * ((static_cast<int64_t>(N) + 255) / 256) >= kWave8MinTiles;
        // small grids take the key split, by the same rule as bf16 inputs
        const int64_t ks_wgs = static_cast<int64_t>(B) * H * ((static_cast<int64_t>(N) + 31) / 32);
        const bool small = N >= kKeySplitMinN && ks_wgs <= (d == 64 ? kKeySplitMaxWgsD64 : kKeySplitMaxWgsD128);
        int bm = 0, threads = 0;
        const Kernel kern = fa::pick_fp8_kernel(d, mask_kind, out_dtype == FA_DTYPE_F32, wide && !small, small, &bm, &threads);
        L = {kern, bm, !small, threads};   // the key split runs single 32-row blocks, never tile pairs
    } else if (in_dtype == FA_DTYPE_BF16) {
        const bool of32 = out_dtype == FA_DTYPE_F32;
        if (d == 64) L = of32 ? pick_bf16_mask<64, true>(mask_kind, variant) : pick_bf16_mask<64, false>(mask_kind, variant);
        else L = of32 ? pick_bf16_mask<128, true>(mask_kind, variant) : pick_bf16_mask<128, false>(mask_kind, variant);
    } else {
        L = d == 64 ? pick_f32_mask<64>(mask_kind) : pick_f32_mask<128>(mask_kind);
    }

    // sizes: element offsets are 64-bit in the kernels; workgroup counts and per-head byte
    // sizes (buffer resources) must fit in 32 bits
    if (!L.kern || L.bm <= 0) return FA_ERR_UNSUPPORTED;
    const int64_t n_qtiles = (static_cast<int64_t>(N) + L.bm - 1) / L.bm;
    const bool causal = (mask_kind & FA_MASK_CAUSAL) != 0;
    const int64_t n_items = (L.paired && causal) ? (n_qtiles + 1) / 2 : n_qtiles;
    const int64_t total = static_cast<int64_t>(B) * H * n_items;
    if (total > 0x7fffffff || static_cast<int64_t>(B) * H > 0x7fffffff) return FA_ERR_INVALID_ARG;
    if (static_cast<int64_t>(N) * d * 4 > 0x7fffffff) return FA_ERR_INVALID_ARG;
    const size_t in_bytes = static_cast<size_t>(B) * H * N * d * (in_dtype == FA_DTYPE_F32 ? 4 : f8 ? 1 : 2);
    const size_t out_bytes = static_cast<size_t>(B) * H * N * d * (out_dtype == FA_DTYPE_F32 ? 4 : 2);
    if (overlaps(o, out_bytes, q, in_bytes) || overlaps(o, out_bytes, k, in_bytes) ||
        overlaps(o, out_bytes, v, in_bytes))
        return FA_ERR_INVALID_ARG;
    if (lse && (overlaps(lse, static_cast<size_t>(B) * H * N * 4, o, out_bytes) ||
                overlaps(lse, static_cast<size_t>(B) * H * N * 4, q, in_bytes) ||
                overlaps(lse, static_cast<size_t>(B) * H * N * 4, k, in_bytes) ||
                overlaps(lse, static_cast<size_t>(B) * H * N * 4, v, in_bytes)))
        return FA_ERR_INVALID_ARG;

    fa::FwdArgs args{};
    args.q = q;
    args.k = k;
    args.v = v;
    args.o = o;
    args.lse = lse;
    args.seqlens = (mask_kind & FA_MASK_KEY_PADDING) ? seqlens : nullptr;
    if (drop) {
        const int t = drop_threshold(drop->p);
        args.drop_k0 = static_cast<uint32_t>(drop->seed);
        args.drop_k1 = static_cast<uint32_t>(drop->seed >> 32);
        args.drop_offset = drop->offset;
        args.drop_t = static_cast<uint32_t>(t);
        args.drop_keep_scale = static_cast<float>(256.0 / (256 - t));
    }
    args.B = B;
    args.H = H;
    args.N = N;
    args.n_qtiles = static_cast<int>(n_qtiles);
    args.total_wgs = static_cast<int>(total);
    args.scale = static_cast<float>(eff_scale);
    args.scale_log2 = static_cast<float>(eff_scale * 1.4426950408889634074);
    args.v_descale = static_cast<float>(dv);

    if (!L.kern) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(L.kern, dim3(static_cast<unsigned>(total)), dim3(L.threads), 0,
                       static_cast<hipStream_t>(stream), args);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return FA_ERR_HIP;
    }
    return FA_OK;
}

using BwdKernel = void (*)(fa::BwdArgs);

template <int D, bool DROP>
void pick_bwd(int mask_kind, BwdKernel& dkdv, BwdKernel& dq) {
    switch (mask_kind) {
        case 0: dkdv = fa::fa_bwd_dkdv_kernel<D, false, false, DROP>; dq = fa::fa_bwd_dq_kernel<D, false, false, DROP>; break;
        case 1: dkdv = fa::fa_bwd_dkdv_kernel<D, true, false, DROP>; dq = fa::fa_bwd_dq_kernel<D, true, false, DROP>; break;
        case 2: dkdv = fa::fa_bwd_dkdv_kernel<D, false, true, DROP>; dq = fa::fa_bwd_dq_kernel<D, false, true, DROP>; break;
        default: dkdv = fa::fa_bwd_dkdv_kernel<D, true, true, DROP>; dq = fa::fa_bwd_dq_kernel<D, true, true, DROP>; break;
    }
}

bool launched_ok() {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return false;
    }
    return true;
}

int bwd_launch(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               float* delta, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
               int mask_kind, const int32_t* seqlens, int in_dtype, int grad_dtype, void* stream,
               const DropSpec* drop = nullptr) {
    // ---- validation (host only, before any HIP call) ----
    if (B < 0 || H < 0 || N < 0) return FA_ERR_INVALID_ARG;
    if (mask_kind < 0 || mask_kind > (FA_MASK_CAUSAL | FA_MASK_KEY_PADDING)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
    if (in_dtype != FA_DTYPE_F32 && in_dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (grad_dtype != FA_DTYPE_F32 && grad_dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (d <= 0) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (in_dtype != FA_DTYPE_BF16 || grad_dtype != FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
    if (drop && drop_threshold(drop->p) < 0) return FA_ERR_INVALID_ARG;
    if (B == 0 || H == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o || !lse || !dout || !delta || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
    if ((mask_kind & FA_MASK_KEY_PADDING) && !seqlens) return FA_ERR_INVALID_ARG;
    const void* t16[] = {q, k, v, o, dout, dq, dk, dv};
    for (const void* p : t16)
        if (!aligned(p, 16)) return FA_ERR_INVALID_ARG;
    if (!aligned(lse, 4) || !aligned(delta, 4)) return FA_ERR_INVALID_ARG;
    if ((mask_kind & FA_MASK_KEY_PADDING) && !aligned(seqlens, 4)) return FA_ERR_INVALID_ARG;
    // sizes: element offsets are 64-bit in the kernels; workgroup counts must fit in 32 bits
    const int64_t bh = static_cast<int64_t>(B) * H;
    const int64_t n_blk = (static_cast<int64_t>(N) + 127) / 128;
    if (bh * n_blk > 0x7fffffff || bh * N / 8 + 1 > 0x7fffffff) return FA_ERR_INVALID_ARG;
    // outputs (the gradients and the workspace) must not overlap each other or any input
    const size_t in_b = static_cast<size_t>(bh) * N * d * 2, g_b = static_cast<size_t>(bh) * N * d * 4;
    const size_t row_b = static_cast<size_t>(bh) * N * 4;
    const void* outs[] = {dq, dk, dv, delta};
    const size_t out_sz[] = {g_b, g_b, g_b, row_b};
    const void* ins[] = {q, k, v, o, dout, lse};
    const size_t in_sz[] = {in_b, in_b, in_b, in_b, in_b, row_b};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return FA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return FA_ERR_INVALID_ARG;
    }

    fa::BwdArgs args{};
    args.q = q;
    args.k = k;
    args.v = v;
    args.o = o;
    args.dout = dout;
    args.lse = lse;
    args.delta = delta;
    args.dq = static_cast<float*>(dq);
    args.dk = static_cast<float*>(dk);
    args.dv = static_cast<float*>(dv);
    args.seqlens = (mask_kind & FA_MASK_KEY_PADDING) ? seqlens : nullptr;
    args.B = B;
    args.H = H;
    args.N = N;
    args.scale = scale;
    args.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
    if (drop) {
        const int t = drop_threshold(drop->p);
        args.drop_k0 = static_cast<uint32_t>(drop->seed);
        args.drop_k1 = static_cast<uint32_t>(drop->seed >> 32);
        args.drop_offset = drop->offset;
        args.drop_t = static_cast<uint32_t>(t);
        args.drop_keep_scale = static_cast<float>(256.0 / (256 - t));
    }

    BwdKernel dkdv, dqk;
    void (*delta_k)(fa::BwdArgs);
    if (d == 64) {
        if (drop) pick_bwd<64, true>(mask_kind, dkdv, dqk);
        else pick_bwd<64, false>(mask_kind, dkdv, dqk);
        delta_k = fa::fa_bwd_delta_kernel<64>;
    } else {
        if (drop) pick_bwd<128, true>(mask_kind, dkdv, dqk);
        else pick_bwd<128, false>(mask_kind, dkdv, dqk);
        delta_k = fa::fa_bwd_delta_kernel<128>;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t rows_per_blk = 256 / (d / 8);
    hipLaunchKernelGGL(delta_k, dim3(static_cast<unsigned>((bh * N + rows_per_blk - 1) / rows_per_blk)),
                       dim3(kThreads), 0, st, args);
    if (!launched_ok()) return FA_ERR_HIP;
    hipLaunchKernelGGL(dkdv, dim3(static_cast<unsigned>(bh * n_blk)), dim3(kThreads), 0, st, args);
    if (!launched_ok()) return FA_ERR_HIP;
    hipLaunchKernelGGL(dqk, dim3(static_cast<unsigned>(bh * n_blk)), dim3(kThreads), 0, st, args);
    if (!launched_ok()) return FA_ERR_HIP;
    return FA_OK;
}

// ---- packed variable-length sequences ------------------------------------------------------

// Query sequences of at most this many rows take the split-key decoding kernel; longer ones the
// pipelined tile kernel.
constexpr int kDecodeMaxRows = 4;
// Workgroups the decoding kernel aims for (8 per CU), and the fewest keys per range.
constexpr int64_t kDecodeTargetWgs = 2048;
constexpr int64_t kDecodeMinKeys = 512;
// Tile kernel on packed sequences: fewest tiles (over all sequences and heads, counted at the
// longest query sequence) for which causal tiles are paired.
constexpr int64_t kPairMinTiles = 4096;

struct DecodePlan {
    int g;            // query rows per sequence the kernel handles (0: not a decoding shape)
    int n_splits;     // key ranges per (sequence, head)
    int chunk;        // keys per range
    size_t ws_bytes;  // workspace for the partial states (0 with one range)
};

// A pure function of the sizes, so the caller can size the workspace before the call.
DecodePlan decode_plan(int B, int H, int max_q, int max_k, int d) {
    DecodePlan p{0, 1, 0, 0};
    if (max_q <= 0 || max_q > kDecodeMaxRows || B <= 0 || H <= 0 || max_k < 0 || (d != 64 && d != 128)) return p;
    p.g = max_q == 1 ? 1 : kDecodeMaxRows;
    const int64_t step = d == 128 ? fa::dec_keys_per_step<128>() : fa::dec_keys_per_step<64>();
    const int64_t bh = static_cast<int64_t>(B) * H;
    int64_t S = (kDecodeTargetWgs + bh - 1) / bh;
    const int64_t smax = (max_k + kDecodeMinKeys - 1) / kDecodeMinKeys;
    S = S < smax ? S : smax;
    S = S < 1 ? 1 : S;
    int64_t chunk = (max_k + S - 1) / S;
    chunk = (chunk + step - 1) / step * step;
    if (chunk < step) chunk = step;
    S = (max_k + chunk - 1) / chunk;
    if (S < 1) S = 1;
    if (S > fa::kDecodeMaxSplits) return DecodePlan{0, 1, 0, 0};   // not reached: S <= kDecodeTargetWgs
    p.n_splits = static_cast<int>(S);
    p.chunk = static_cast<int>(chunk);
    p.ws_bytes = S > 1 ? static_cast<size_t>(bh) * S * p.g * (d + 2) * sizeof(float) : 0;
    return p;
}

// Packed prefill whose tiles give at most half a workgroup per compute unit (the tile kernel
// runs two) splits each (sequence, head)'s keys into ranges so that the grid reaches about two
// workgroups per CU; ranges hold at least kSplitMinKeys keys.  Measured: one 4096-token
// sequence, d=64, 58 -> 23 us; one 8192-token sequence with two heads, d=128 causal, 160 -> 73
// us.  With one workgroup per CU (chunked_prefill: 256 tiles) the split kernel gained 4 % and
// its merge took it back, so those grids stay unsplit.
constexpr int64_t kSplitMaxTileWgs = 128;
constexpr int64_t kSplitTargetWgs = 512;
constexpr int kSplitMinKeys = 512;
constexpr int kSplitMaxRanges = 16;

struct VarlenPlan {
    DecodePlan dec;   // decoding shapes (dec.g > 0)
    int S;            // key ranges of the split tile kernel (1: no split)
    int chunk;        // keys per range
    size_t ws_bytes;  // workspace of whichever path runs
};

// A pure function of the sizes (and of the most workspace the caller can give: the
// allocation-free entry point passes its fixed array's size and then runs unsplit instead).
VarlenPlan varlen_plan(int B, int H, int max_q, int max_k, int d, size_t ws_limit) {
    VarlenPlan p{decode_plan(B, H, max_q, max_k, d), 1, 0, 0};
    if (p.dec.g > 0) {
        p.ws_bytes = p.dec.ws_bytes;
        return p;
    }
    if (B <= 0 || H <= 0 || max_q <= 0 || max_k < 2 * kSplitMinKeys || (d != 64 && d != 128)) return p;
    const int64_t bh = static_cast<int64_t>(B) * H;
    const int64_t tiles = bh * ((static_cast<int64_t>(max_q) + 127) / 128);
    if (tiles > kSplitMaxTileWgs) return p;
    int64_t S = (kSplitTargetWgs + tiles - 1) / tiles;
    const int64_t smax = max_k / kSplitMinKeys;
    S = S < smax ? S : smax;
    S = S < kSplitMaxRanges ? S : kSplitMaxRanges;
    if (S < 2) return p;
    int64_t chunk = (max_k + S - 1) / S;
    chunk = (chunk + 63) / 64 * 64;
    S = (max_k + chunk - 1) / chunk;
    if (S < 2) return p;
    const size_t ws = static_cast<size_t>(S) * bh * max_q * (d + 1) * sizeof(float);
    if (ws > ws_limit) return p;
    p.S = static_cast<int>(S);
    p.chunk = static_cast<int>(chunk);
    p.ws_bytes = ws;
    return p;
}

template <int D, bool OUTF32>
Kernel pick_varlen_split(bool causal) {
    return causal ? fa::fa_fwd_bf16_varlen_split_kernel<D, 64, true, OUTF32> : fa::fa_fwd_bf16_varlen_split_kernel<D, 64, false, OUTF32>;
}

template <int D, bool OUTF32>
Kernel pick_varlen(bool causal) {
    return causal ? fa::fa_fwd_bf16_varlen_kernel<D, 64, 1, true, OUTF32> : fa::fa_fwd_bf16_varlen_kernel<D, 64, 1, false, OUTF32>;
}

using DecKernel = void (*)(fa::DecArgs);

template <int D, bool OUTF32>
void pick_decode(int g, bool causal, DecKernel& main, DecKernel& merge) {
    if (g == 1) {
        main = causal ? fa::fa_decode_kernel<D, 1, true, OUTF32> : fa::fa_decode_kernel<D, 1, false, OUTF32>;
        merge = fa::fa_decode_merge_kernel<D, 1, OUTF32>;
    } else {
        main = causal ? fa::fa_decode_kernel<D, kDecodeMaxRows, true, OUTF32>
                      : fa::fa_decode_kernel<D, kDecodeMaxRows, false, OUTF32>;
        merge = fa::fa_decode_merge_kernel<D, kDecodeMaxRows, OUTF32>;
    }
}

int varlen_launch(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_q,
                  const int32_t* cu_k, int B, int H, int total_q, int total_k, int max_q, int max_k, int d,
                  float scale, int mask_kind, int causal_align, void* workspace, size_t workspace_bytes,
                  int in_dtype, int out_dtype, void* stream, bool use_scratch = false) {
    // ---- validation (host only, before any HIP call) ----
    if (B < 0 || H < 0 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0) return FA_ERR_INVALID_ARG;
    if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL) return FA_ERR_INVALID_ARG;
    if (causal_align != FA_ALIGN_BOTTOM_RIGHT && causal_align != FA_ALIGN_TOP_LEFT) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
    if (in_dtype != FA_DTYPE_F32 && in_dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (out_dtype != FA_DTYPE_F32 && out_dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (d <= 0) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (in_dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || total_q == 0 || max_q == 0) return FA_OK;
    if (!q || !o || !cu_q || !cu_k) return FA_ERR_INVALID_ARG;
    if (total_k > 0 && (!k || !v)) return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(o, 16) || (k && !aligned(k, 16)) || (v && !aligned(v, 16))) return FA_ERR_INVALID_ARG;
    if ((lse && !aligned(lse, 4)) || !aligned(cu_q, 4) || !aligned(cu_k, 4)) return FA_ERR_INVALID_ARG;
    // a key range's byte span must fit the 32-bit range of a buffer resource
    const int64_t row_bytes = static_cast<int64_t>(H) * d * 2;
    if (static_cast<int64_t>(max_k) * row_bytes > 0xffffffffLL) return FA_ERR_INVALID_ARG;
    const bool causal = mask_kind == FA_MASK_CAUSAL;
    const VarlenPlan vplan = varlen_plan(B, H, max_q, max_k, d, use_scratch ? kScratchBytes : static_cast<size_t>(-1));
    const DecodePlan& dplan = vplan.dec;
    struct { size_t ws_bytes; int n_splits; } plan{vplan.ws_bytes, dplan.n_splits};
    // the allocation-free entry point takes the library's fixed per-device array as the
    // workspace (its address is fetched after every check has passed)
    const bool from_scratch = use_scratch && plan.ws_bytes > 0;
    if (from_scratch && plan.ws_bytes > kScratchBytes) return FA_ERR_SCRATCH_LIMIT;
    if (plan.ws_bytes > 0 && !from_scratch) {
        if (!workspace || workspace_bytes < plan.ws_bytes || !aligned(workspace, 16)) return FA_ERR_INVALID_ARG;
    }
    const int64_t bh = static_cast<int64_t>(B) * H;
    const int64_t n_qtiles = (static_cast<int64_t>(max_q) + 127) / 128;
    // causal tiles are paired (equal work per item) only when the pairs still fill the chip
    // several times over; otherwise every tile is its own work item
    const bool pair = causal && bh * n_qtiles >= kPairMinTiles;
    const int64_t items = pair ? (n_qtiles + 1) / 2 : n_qtiles;
    // tile kernel grid: head bh on XCD bh % 8, so the head count is rounded up to a multiple of 8
    // (split: each (head, key range) pair counts as a head)
    const int64_t tile_wgs = (bh * vplan.S + fa::kNumXcd - 1) / fa::kNumXcd * fa::kNumXcd * items;
    const int64_t merge_blocks = (bh * max_q * (d / 4) + 255) / 256;
    if (tile_wgs > 0x7fffffff || bh * plan.n_splits > 0x7fffffff || bh * kDecodeMaxRows > 0x7fffffff ||
        merge_blocks > 0x7fffffff)
        return FA_ERR_INVALID_ARG;
    // outputs must not overlap each other or any input
    const size_t qb = static_cast<size_t>(total_q) * H * d * 2, kb = static_cast<size_t>(total_k) * H * d * 2;
    const size_t ob = static_cast<size_t>(total_q) * H * d * (out_dtype == FA_DTYPE_F32 ? 4 : 2);
    const size_t lb = static_cast<size_t>(total_q) * H * 4;
    const size_t cb = (static_cast<size_t>(B) + 1) * 4;
    const void* ins[] = {q, k, v, cu_q, cu_k};
    const size_t in_sz[] = {qb, kb, kb, cb, cb};
    const void* outs[] = {o, lse, plan.ws_bytes ? workspace : nullptr};
    const size_t out_sz[] = {ob, lb, plan.ws_bytes};
    for (int i = 0; i < 3; ++i) {
        if (!outs[i]) continue;
        for (int j = 0; j < 5; ++j)
            if (ins[j] && overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return FA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 3; ++j)
            if (outs[j] && overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return FA_ERR_INVALID_ARG;
    }
    if (from_scratch) {
        const int status = scratch_on_current_device(&workspace);
        if (status != FA_OK) return status;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
    const bool of32 = out_dtype == FA_DTYPE_F32;

    if (dplan.g > 0) {
        fa::DecArgs a;
        a.q = q;
        a.k = k;
        a.v = v;
        a.o = o;
        a.lse = lse;
        a.cu_q = cu_q;
        a.cu_k = cu_k;
        a.ws = static_cast<float*>(plan.ws_bytes ? workspace : nullptr);
        a.B = B;
        a.H = H;
        a.total_q = total_q;
        a.total_k = total_k;
        a.max_q = max_q;
        a.max_k = max_k;
        a.n_splits = dplan.n_splits;
        a.chunk = dplan.chunk;
        a.bottom_right = causal_align == FA_ALIGN_BOTTOM_RIGHT;
        a.scale_log2 = scale_log2;
        DecKernel main, merge;
        if (d == 64) {
            if (of32) pick_decode<64, true>(dplan.g, causal, main, merge);
            else pick_decode<64, false>(dplan.g, causal, main, merge);
        } else {
            if (of32) pick_decode<128, true>(dplan.g, causal, main, merge);
            else pick_decode<128, false>(dplan.g, causal, main, merge);
        }
        hipLaunchKernelGGL(main, dim3(static_cast<unsigned>(bh * plan.n_splits)), dim3(kThreads), 0, st, a);
        if (!launched_ok()) return FA_ERR_HIP;
        if (dplan.n_splits > 1) {
            const int64_t merge_wgs = bh * dplan.g * (d / fa::kMergeCols);
            hipLaunchKernelGGL(merge, dim3(static_cast<unsigned>(merge_wgs)), dim3(kThreads), 0, st, a);
            if (!launched_ok()) return FA_ERR_HIP;
        }
        return FA_OK;
    }

    fa::FwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.seqlens = nullptr;
    a.B = B;
    a.H = H;
    a.N = 0;
    a.n_qtiles = static_cast<int>(n_qtiles);
    a.total_wgs = static_cast<int>(tile_wgs);
    a.scale = scale;
    a.scale_log2 = scale_log2;
    a.cu_q = cu_q;
    a.cu_k = cu_k;
    a.total_q = total_q;
    a.total_k = total_k;
    a.max_q = max_q;
    a.max_k = max_k;
    a.bottom_right = causal_align == FA_ALIGN_BOTTOM_RIGHT;
    a.pair = pair ? 1 : 0;
    if (vplan.S > 1) {
        // key ranges into the workspace, then their merge into O and LSE
        a.ws_o = static_cast<float*>(workspace);
        a.ws_lse = a.ws_o + static_cast<size_t>(vplan.S) * bh * max_q * d;
        a.n_ranges = vplan.S;
        a.range_keys = vplan.chunk;
        Kernel kern, merge;
        if (d == 64) {
            kern = of32 ? pick_varlen_split<64, true>(causal) : pick_varlen_split<64, false>(causal);
            merge = of32 ? fa::fa_fwd_varlen_merge_kernel<64, true> : fa::fa_fwd_varlen_merge_kernel<64, false>;
        } else {
            kern = of32 ? pick_varlen_split<128, true>(causal) : pick_varlen_split<128, false>(causal);
            merge = of32 ? fa::fa_fwd_varlen_merge_kernel<128, true> : fa::fa_fwd_varlen_merge_kernel<128, false>;
        }
        hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tile_wgs)), dim3(kThreads), 0, st, a);
        if (!launched_ok()) return FA_ERR_HIP;
        hipLaunchKernelGGL(merge, dim3(static_cast<unsigned>(merge_blocks)), dim3(kThreads), 0, st, a);
        if (!launched_ok()) return FA_ERR_HIP;
        return FA_OK;
    }
    Kernel kern;
    if (d == 64) kern = of32 ? pick_varlen<64, true>(causal) : pick_varlen<64, false>(causal);
    else kern = of32 ? pick_varlen<128, true>(causal) : pick_varlen<128, false>(causal);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tile_wgs)), dim3(kThreads), 0, st, a);
    if (!launched_ok()) return FA_ERR_HIP;
    return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_fwd_varlen_workspace_size(int B, int H, int max_seqlen_q, int max_seqlen_k, int d) {
    return varlen_plan(B, H, max_seqlen_q, max_seqlen_k, d, static_cast<size_t>(-1)).ws_bytes;
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int B, int H, int total_q, int total_k, int max_seqlen_q,
                  int max_seqlen_k, int d, float scale, int mask_kind, int causal_align, void* workspace,
                  size_t workspace_bytes, int in_dtype, int out_dtype, void* stream) {
    return varlen_launch(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k, max_seqlen_q,
                         max_seqlen_k, d, scale, mask_kind, causal_align, workspace, workspace_bytes, in_dtype,
                         out_dtype, stream);
}

int fa_fwd_varlen_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, int B, int H, int total_q, int total_k, int max_seqlen_q,
                          int max_seqlen_k, int d, float scale, int mask_kind, int causal_align, int in_dtype,
                          int out_dtype, void* stream) {
    return varlen_launch(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k, max_seqlen_q,
                         max_seqlen_k, d, scale, mask_kind, causal_align, nullptr, 0, in_dtype, out_dtype, stream,
                         true);
}

size_t fa_scratch_bytes(void) { return kScratchBytes; }

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           float* delta, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int mask_kind,
           const int32_t* seqlens, int in_dtype, int grad_dtype, void* stream) {
    return bwd_launch(q, k, v, o, lse, dout, delta, dq, dk, dv, B, H, N, d, scale, mask_kind, seqlens, in_dtype,
                      grad_dtype, stream);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   float* delta, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int mask_kind,
                   const int32_t* seqlens, float p_drop, uint64_t seed, uint32_t offset, int in_dtype, int grad_dtype,
                   void* stream) {
    const DropSpec drop{p_drop, seed, offset};
    return bwd_launch(q, k, v, o, lse, dout, delta, dq, dk, dv, B, H, N, d, scale, mask_kind, seqlens, in_dtype,
                      grad_dtype, stream, &drop);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int mask_kind, const int32_t* seqlens, int in_dtype, int out_dtype,
           void* stream) {
    return launch(q, k, v, o, lse, B, H, N, d, scale, mask_kind, seqlens, in_dtype, out_dtype, stream, 0);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int mask_kind, const int32_t* seqlens, float p_drop, uint64_t seed, uint32_t offset,
                   int in_dtype, int out_dtype, void* stream) {
    const DropSpec drop{p_drop, seed, offset};
    return launch(q, k, v, o, lse, B, H, N, d, scale, mask_kind, seqlens, in_dtype, out_dtype, stream, 0, &drop);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, float descale_q, float descale_k, float descale_v, int mask_kind, const int32_t* seqlens,
               int out_dtype, void* stream) {
    const float descale[3] = {descale_q, descale_k, descale_v};
    return launch(q, k, v, o, lse, B, H, N, d, scale, mask_kind, seqlens, FA_DTYPE_FP8_E4M3, out_dtype, stream, 0,
                  nullptr, descale);
}

int fa_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, float scale, int mask_kind, const int32_t* seqlens, int in_dtype,
                   int out_dtype, void* stream, int variant) {
    return launch(q, k, v, o, lse, B, H, N, d, scale, mask_kind, seqlens, in_dtype, out_dtype, stream,
                  variant);
}

int fa_variant_count(void) { return kNumVariants; }

const char* fa_status_str(int status) {
    switch (status) {
        case FA_OK: return "FA_OK: success";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: no kernel for this head width, dtype pair or variant";
        case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed (see fa_last_hip_error)";
        case FA_ERR_SCRATCH_LIMIT:
            return "FA_ERR_SCRATCH_LIMIT: the call needs more workspace than the library's fixed scratch holds "
                   "(use the entry point that takes a caller workspace)";
        default: return "unknown fa_status";
    }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

int fa_version(void) { return FA_VERSION; }

}  // extern "C"
