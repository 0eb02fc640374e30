// Decoding-shaped exact attention for bf16 inputs on gfx950 (MI355X): at most a few query rows
// per sequence against a long key range, for packed token-major [T, H, d] tensors.
//
// With one (or a handful of) query rows the work is a matrix-vector product per key tile: two
// FLOP per byte of K and V, far below the MFMA units' break-even, so the kernel is bound by the
// HBM stream of K and V and is written for that -- plain vector loads of whole 256-byte rows,
// fp32 vector arithmetic, no matrix cores and no LDS staging of the stream.  The prefill and
// decode shapes differ in query shape and data reuse ("FlashAttention Interview Questions: IO
// Complexity, Tiling, and Numerical Stability", closing benchmark section), hence a separate
// kernel.
//
// A sequence's keys are cut into `n_splits` ranges handled by independent workgroups, so a
// small batch still fills the chip.  Every workgroup keeps the running statistics of the
// page's section "How can softmax be computed across tiles?" (running maximum m, shifted sum l,
// unnormalised accumulator a) over its range, in base 2 on scores pre-multiplied by
// scale*log2(e).  With one range it writes O = a / l and the log-sum-exp directly; otherwise it
// writes (m, l, a) to the caller's workspace and fa_decode_merge_kernel combines the ranges
// with the same rescaling, exp2(m_r - max_r m_r).
//
// Layout inside a workgroup (4 wave64s): a key row of d bf16 values is read by LPK = d/8 lanes,
// 16 bytes each, so one wave instruction moves KPW = 64/LPK whole rows; each lane keeps its 8
// columns of the query rows and of the accumulators.  The row dot product is reduced across
// the LPK lanes with DPP row operations.  Every (wave, lane group) runs its own statistics
// over an interleaved subset of the keys; the 4*KPW partial states are combined through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_bf16.h"

namespace fa {

struct DecArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* cu_q;
    const int32_t* cu_k;
    float* ws;             // n_splits > 1: partial accumulators, then partial (m, l)
    int B, H;
    int total_q, total_k;
    int max_q, max_k;
    int n_splits;          // key ranges per (sequence, head)
    int chunk;             // keys per range (a multiple of the keys one workgroup step covers)
    int bottom_right;      // causal alignment: 1 bottom-right, 0 top-left
    float scale_log2;      // scale * log2(e)
};

// Sum over each group of 8 (D = 64) or 16 (D = 128) consecutive lanes, result in every lane of
// the group.  DPP row operations act within 16-lane rows; half_mirror / mirror pair lane i with
// 7-i / 15-i, after which two quad permutations finish the sum.
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
    auto dpp = [](float v, auto ctrl_c) __attribute__((always_inline)) {
        constexpr int CTRL = decltype(ctrl_c)::value;
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
    };
    if constexpr (LPK == 16) x += dpp(x, std::integral_constant<int, 0x140>{});   // row_mirror
    x += dpp(x, std::integral_constant<int, 0x141>{});                            // row_half_mirror
    x += dpp(x, std::integral_constant<int, 0x4E>{});                             // quad_perm [2,3,0,1]
    x += dpp(x, std::integral_constant<int, 0xB1>{});                             // quad_perm [1,0,3,2]
    return x;
}

__device__ __forceinline__ float bf16_to_f32_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_to_f32_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Keys one workgroup covers per step: 4 waves x KPW rows x U rows in flight per lane group.
template <int D>
constexpr int dec_keys_per_step() { return 4 * (64 / (D / 8)) * 4; }

// One workgroup per (sequence, head, key range).  G: query rows handled (the launch's longest
// query sequence is at most G).
template <int D, int G, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(256) fa_decode_kernel(DecArgs a) {
    constexpr int LPK = D / 8;             // lanes per key row
    constexpr int KPW = 64 / LPK;          // key rows per wave instruction
    constexpr int U = 4;                   // key rows in flight per lane group
    constexpr int NGRP = 4 * KPW;          // independent partial states per workgroup
    constexpr int STEP = dec_keys_per_step<D>();

    __shared__ float sm_acc[NGRP][G][D];
    __shared__ float sm_m[NGRP][G];
    __shared__ float sm_l[NGRP][G];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kg = lane / LPK;             // key row of the wave instruction
    const int e0 = (lane % LPK) * 8;       // this lane's 8 columns
    const int grp = wave * KPW + kg;

    const int split = blockIdx.x % a.n_splits;
    const int bh = blockIdx.x / a.n_splits;
    const int b = bh / a.H;
    const int h = bh - b * a.H;

    auto clampi = [](int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); };
    const int qs = clampi(a.cu_q[b], 0, a.total_q);
    const int qe = clampi(a.cu_q[b + 1], qs, a.total_q);
    const int ks = clampi(a.cu_k[b], 0, a.total_k);
    const int ke = clampi(a.cu_k[b + 1], ks, a.total_k);
    int Lq = qe - qs < a.max_q ? qe - qs : a.max_q;
    Lq = Lq < G ? Lq : G;
    const int Lk = ke - ks < a.max_k ? ke - ks : a.max_k;
    if (Lq <= 0) return;                   // uniform over the workgroup
    const int dlt = a.bottom_right ? Lk - Lq : 0;
    const int RSE = a.H * D;               // elements between consecutive token rows

    // key range of this workgroup, cut at the last key any of its rows may see
    const int k_lo = split * a.chunk;
    int k_hi = k_lo + a.chunk < Lk ? k_lo + a.chunk : Lk;
    if (CAUSAL) k_hi = k_hi < Lq + dlt ? k_hi : Lq + dlt;

    // query rows (8 columns per lane), pre-multiplied by scale * log2(e)
    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int r = g < Lq ? g : Lq - 1;
        const u32x4 w = *(const u32x4*)((const uint16_t*)a.q + ((int64_t)(qs + r) * a.H + h) * D + e0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            qv[g][2 * t] = bf16_to_f32_lo(w[t]) * a.scale_log2;
            qv[g][2 * t + 1] = bf16_to_f32_hi(w[t]) * a.scale_log2;
        }
    }

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }

    const uint16_t* kp = (const uint16_t*)a.k + ((int64_t)ks * a.H + h) * D + e0;
    const uint16_t* vp = (const uint16_t*)a.v + ((int64_t)ks * a.H + h) * D + e0;
    for (int kb = k_lo; kb < k_hi; kb += STEP) {
        // issue all loads of the step first: U rows of K and of V per lane group
        u32x4 kr[U], vr[U];
        int key[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            key[u] = kb + (u * 4 + wave) * KPW + kg;
            kr[u] = u32x4{0u, 0u, 0u, 0u};
            vr[u] = u32x4{0u, 0u, 0u, 0u};
            if (key[u] < k_hi) {
                kr[u] = __builtin_nontemporal_load((const u32x4*)(kp + (int64_t)key[u] * RSE));
                vr[u] = __builtin_nontemporal_load((const u32x4*)(vp + (int64_t)key[u] * RSE));
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float s[U];
            float mx = m[g];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float part = 0.f;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    part = fmaf(qv[g][2 * t], bf16_to_f32_lo(kr[u][t]), part);
                    part = fmaf(qv[g][2 * t + 1], bf16_to_f32_hi(kr[u][t]), part);
                }
                part = group_sum<LPK>(part);
                const bool ok = key[u] < k_hi && (!CAUSAL || key[u] <= g + dlt);
                s[u] = ok ? part : kNegInf;
                mx = __builtin_elementwise_maximum(mx, s[u]);
            }
            if (mx == kNegInf) continue;   // no visible key for this row yet (uniform per group)
            const float alpha = fast_exp2(m[g] - mx);   // m = -inf before the first key: 0
            m[g] = mx;
            float p[U];
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u] = fast_exp2(s[u] - mx);
                psum += p[u];
            }
            l[g] = fmaf(l[g], alpha, psum);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    acc[g][2 * t] = fmaf(p[u], bf16_to_f32_lo(vr[u][t]), acc[g][2 * t]);
                    acc[g][2 * t + 1] = fmaf(p[u], bf16_to_f32_hi(vr[u][t]), acc[g][2 * t + 1]);
                }
        }
    }

    // combine the NGRP partial states of the workgroup
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_acc[grp][g][e0 + e] = acc[g][e];
        if (lane % LPK == 0) {
            sm_m[grp][g] = m[g];
            sm_l[grp][g] = l[g];
        }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += 256) {
        const int g = i / D, e = i % D;
        if (g >= Lq) continue;
        float M = kNegInf;
#pragma unroll
        for (int r = 0; r < NGRP; ++r) M = __builtin_elementwise_maximum(M, sm_m[r][g]);
        float L = 0.f, A = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int r = 0; r < NGRP; ++r) {
                const float w = fast_exp2(sm_m[r][g] - M);   // -inf partials weigh 0
                L = fmaf(sm_l[r][g], w, L);
                A = fmaf(sm_acc[r][g][e], w, A);
            }
        }
        if (a.n_splits > 1) {
            const int64_t slot = ((int64_t)bh * a.n_splits + split) * G + g;
            a.ws[slot * D + e] = A;
            if (e == 0) {
                float* ml = a.ws + (int64_t)a.B * a.H * a.n_splits * G * D;
                ml[2 * slot] = M;
                ml[2 * slot + 1] = L;
            }
        } else {
            const bool none = !(L > 0.f);
            const int64_t row = (int64_t)(qs + g) * a.H + h;
            const float o = none ? 0.f : A / L;
            if (OUT_F32) ((float*)a.o)[row * D + e] = o;
            else ((__bf16*)a.o)[row * D + e] = (__bf16)o;
            if (e == 0 && a.lse) a.lse[(int64_t)h * a.total_q + qs + g] = none ? kNegInf : (M + __log2f(L)) * kLn2;
        }
    }
}

// Most key ranges one (sequence, head) is cut into (the host caps the split count here).
constexpr int kDecodeMaxSplits = 2048;

// Combine the key ranges of fa_decode_kernel.  One workgroup per (sequence, head, query row,
// slice of MCW output columns): all 256 threads first find the largest range maximum M and
// the weights exp2(m_r - M) (kept in LDS) and the total l; then 256 / MCW groups of threads
// each sum a share of the ranges for the slice's columns, so the partial states are read with
// many loads in flight instead of one range after another.
constexpr int kMergeCols = 16;

template <int D, int G, bool OUT_F32>
__global__ void __launch_bounds__(256) fa_decode_merge_kernel(DecArgs a) {
    constexpr int MCW = kMergeCols;
    constexpr int NCS = D / MCW;           // column slices per row
    constexpr int NSG = 256 / MCW;         // range groups
    __shared__ float wsh[kDecodeMaxSplits];
    __shared__ float red[4];
    __shared__ float part[NSG][MCW];

    const int tid = threadIdx.x;
    const int item = blockIdx.x / NCS;
    const int cs = blockIdx.x - item * NCS;
    const int bh = item / G;
    const int g = item - bh * G;
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    auto clampi = [](int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); };
    const int qs = clampi(a.cu_q[b], 0, a.total_q);
    const int qe = clampi(a.cu_q[b + 1], qs, a.total_q);
    int Lq = qe - qs < a.max_q ? qe - qs : a.max_q;
    Lq = Lq < G ? Lq : G;
    if (g >= Lq) return;                   // uniform over the workgroup

    const int S = a.n_splits;
    const float* ml = a.ws + (int64_t)a.B * a.H * S * G * D;
    auto m_of = [&](int s) { return ml[2 * (((int64_t)bh * S + s) * G + g)]; };
    auto l_of = [&](int s) { return ml[2 * (((int64_t)bh * S + s) * G + g) + 1]; };
    auto block_reduce = [&](float x, bool is_max) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float y = __shfl_xor(x, o);
            x = is_max ? __builtin_elementwise_maximum(x, y) : x + y;
        }
        if ((tid & 63) == 0) red[tid >> 6] = x;
        __syncthreads();
        const float r = is_max ? __builtin_elementwise_maximum(__builtin_elementwise_maximum(red[0], red[1]),
                                                               __builtin_elementwise_maximum(red[2], red[3]))
                               : (red[0] + red[1]) + (red[2] + red[3]);
        __syncthreads();                   // red is reused
        return r;
    };

    float mloc = kNegInf;
    for (int s = tid; s < S; s += 256) mloc = __builtin_elementwise_maximum(mloc, m_of(s));
    const float M = block_reduce(mloc, true);
    float lloc = 0.f;
    for (int s = tid; s < S; s += 256) {
        const float w = M == kNegInf ? 0.f : fast_exp2(m_of(s) - M);   // empty ranges weigh 0
        wsh[s] = w;
        lloc = fmaf(l_of(s), w, lloc);
    }
    const float L = block_reduce(lloc, false);   // its barriers also publish wsh

    const int c = tid % MCW;
    const int sg = tid / MCW;
    const int col = cs * MCW + c;
    const float* accp = a.ws + ((int64_t)bh * S * G + g) * D + col;
    float A = 0.f;
#pragma unroll 8
    for (int s = sg; s < S; s += NSG) A = fmaf(wsh[s], accp[(int64_t)s * G * D], A);
    part[sg][c] = A;
    __syncthreads();
    if (tid < MCW) {
        float t = 0.f;
#pragma unroll
        for (int r = 0; r < NSG; ++r) t += part[r][tid];
        const bool none = !(L > 0.f);
        const int64_t row = (int64_t)(qs + g) * a.H + h;
        const float o = none ? 0.f : t / L;
        if (OUT_F32) ((float*)a.o)[row * D + col] = o;
        else ((__bf16*)a.o)[row * D + col] = (__bf16)o;
        if (cs == 0 && tid == 0 && a.lse) a.lse[(int64_t)h * a.total_q + qs + g] = none ? kNegInf : (M + __log2f(L)) * kLn2;
    }
}

}  // namespace fa
