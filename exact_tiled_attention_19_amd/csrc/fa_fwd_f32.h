// Fused exact-attention forward for float32 inputs and output on gfx950.
//
// Same algorithm and work mapping as the bf16 kernel (one workgroup per (batch, head,
// 128-row query tile), running maximum / sum / accumulator per query row, update of
// "FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical Stability",
// section "How can softmax be computed across tiles?"), but every product is an fp32 MFMA
// (v_mfma_f32_32x32x2_f32) so no operand is ever rounded below float32.
//   * S^T = K Q^T: A operand K[key][2c + hh], B operand Q[query][2c + hh], one float each.
//   * O^T += V^T P^T: the probability in S^T accumulator register r is, for lane half hh,
//     key kappa_hh(r) = 8(r/4) + 4hh + r%4 of the 32-key block; one MFMA per register pairs
//     kappa_0(r) with kappa_1(r), and lane (d, hh) supplies V[kappa_hh(r)][d].
#pragma once

#include "fa_fwd_bf16.h"

namespace fa {

template <int D, bool CAUSAL, bool PAD>
__global__ void __launch_bounds__(256, 2) fa_fwd_f32_kernel(FwdArgs a) {
    constexpr int BM = 128;
    constexpr int BN = 32;
    constexpr int NT = 256;
    constexpr int KC = D / 2;
    constexpr int NDB = D / 32;
    constexpr int STR = D + 4;              // LDS row stride (floats), 16-byte aligned rows
    constexpr int BUF = BN * STR;
    constexpr int CPR = D / 4;              // 16-byte chunks per row
    constexpr int LDC = BN * CPR / NT;
    static_assert(LDC * NT == BN * CPR, "tile must split evenly over the workgroup");

    __shared__ __attribute__((aligned(16))) float smem[4 * BUF];
    float* const kbuf = smem;
    float* const vbuf = smem + 2 * BUF;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const TileCoord tc = tile_of(xcd_remap(blockIdx.x, a.total_wgs), a.n_qtiles, CAUSAL);
    const int b = tc.bh / a.H;
    const int N = a.N;
    const int q0 = tc.qt * BM;
    const int qw0 = q0 + wave * 32;
    const int qrow = qw0 + l32;
    const int64_t base = (int64_t)tc.bh * N * D;

    int Lk = N;
    if (PAD) {
        const int s = a.seqlens[b];
        Lk = s < 0 ? 0 : (s > N ? N : s);
    }
    if (Lk == 0) {
        if (qrow < N) {
            if (hh == 0 && a.lse) a.lse[(int64_t)tc.bh * N + qrow] = kNegInf;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float* op = (float*)a.o + base + (int64_t)qrow * D + 32 * db + 8 * j + 4 * hh;
                    *(f32x4*)op = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
        return;
    }
    int kv_end = Lk;
    if (CAUSAL) kv_end = kv_end < q0 + BM ? kv_end : q0 + BM;
    const int n_tiles = (kv_end + BN - 1) / BN;

    float qf[KC];
    {
        const float* qp = (const float*)a.q + base + (int64_t)(qrow < N ? qrow : N - 1) * D + hh;
#pragma unroll
        for (int c = 0; c < KC; ++c) qf[c] = qrow < N ? qp[2 * c] : 0.f;
    }

    const float* const kg = (const float*)a.k + base;
    const float* const vg = (const float*)a.v + base;
    f32x4 kr[LDC], vr[LDC];
    auto gload = [&](int tile) {
        const int kv0 = tile * BN;
#pragma unroll
        for (int i = 0; i < LDC; ++i) {
            const int ci = tid + NT * i;
            const int row = ci / CPR;
            const int cc = ci - row * CPR;
            int gr = kv0 + row;
            gr = gr < N ? gr : N - 1;
            kr[i] = *(const f32x4*)(kg + (int64_t)gr * D + cc * 4);
            vr[i] = *(const f32x4*)(vg + (int64_t)gr * D + cc * 4);
        }
    };
    auto swrite = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LDC; ++i) {
            const int ci = tid + NT * i;
            const int row = ci / CPR;
            const int cc = ci - row * CPR;
            *(f32x4*)(kbuf + buf * BUF + row * STR + cc * 4) = kr[i];
            *(f32x4*)(vbuf + buf * BUF + row * STR + cc * 4) = vr[i];
        }
    };

    float m_run = kNegInf;
    float l_run = 0.f;
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    gload(0);
    swrite(0);
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int kv0 = t * BN;
        const bool has_next = t + 1 < n_tiles;
        if (has_next) gload(t + 1);
        const float* ks = kbuf + (t & 1) * BUF;
        const float* vs = vbuf + (t & 1) * BUF;
        const bool wave_active = !CAUSAL || kv0 <= qw0 + 31;
        if (wave_active) {
            f32x16 s = f32x16{};
#pragma unroll
            for (int c = 0; c < KC; ++c)
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[l32 * STR + 2 * c + hh], qf[c], s, 0, 0, 0);
            const bool need_mask = (kv0 + BN > Lk) || (CAUSAL && kv0 + BN - 1 > qw0);
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const bool ok = key < Lk && (!CAUSAL || key <= qrow);
                    s[r] = ok ? s[r] : kNegInf;
                }
            }
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = xor32_max(mx);
            const float m_tile = (mx == kNegInf) ? kNegInf : mx * a.scale_log2;
            const float m_new = fmaxf(m_run, m_tile);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], a.scale_log2, -m_use));
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const bool ok = key < Lk && (!CAUSAL || key <= qrow);
                    s[r] = ok ? s[r] : 0.f;
                }
            }
            float rs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) rs += s[r];
            l_run = alpha * l_run + rs;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * STR + 32 * db + l32], s[r], acc[db], 0, 0, 0);
            }
        }
        if (has_next) swrite((t + 1) & 1);
        __syncthreads();
    }

    const float l_tot = xor32_sum(l_run);
    const float inv_l = 1.0f / l_tot;
    if (qrow < N) {
        if (hh == 0 && a.lse) a.lse[(int64_t)tc.bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float* op = (float*)a.o + base + (int64_t)qrow * D + 32 * db + 8 * j + 4 * hh;
                *(f32x4*)op = f32x4{acc[db][4 * j] * inv_l, acc[db][4 * j + 1] * inv_l,
                                    acc[db][4 * j + 2] * inv_l, acc[db][4 * j + 3] * inv_l};
            }
    }
}

}  // namespace fa
