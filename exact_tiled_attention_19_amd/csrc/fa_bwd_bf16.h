// Backward pass of the fused exact-attention forward, bf16 inputs, float32 gradients, gfx950.
//
// What is computed, for one (batch, head) with P = softmax(scale * Q K^T over visible keys):
//     dV = P^T dO,   dP = dO V^T,   D_i = dO_i . O_i,   dS = P * (dP - D),
//     dQ = scale * dS K,   dK = scale * dS^T Q.
// The probabilities are not stored by the forward pass: they are recomputed tile by tile from
// Q, K and the saved log-sum-exp, p_ij = exp(scale * q_i . k_j - LSE_i) ("FlashAttention
// Interview Questions: IO Complexity, Tiling, and Numerical Stability", section "Why can
// recomputation help training?"), so no N x N buffer exists here either.  exp is taken base 2
// on scores pre-multiplied by scale*log2(e) and LSE*log2(e), which is the same function.
//
// Three kernels, all on one stream, none with atomics (the result is run-to-run identical):
//   fa_bwd_delta_kernel  D_i = dO_i . O_i for every row, into the caller's float32 workspace.
//   fa_bwd_dkdv_kernel   one workgroup per (batch, head, 128 keys), 32 keys per wave; the
//                        wave's K^T and V^T stay in VGPRs while 32-row tiles of Q and dO stream
//                        through LDS.  Per tile: S = Q K^T and dP = dO V^T (MFMA, A from LDS,
//                        B from VGPRs); P and dS elementwise; dV^T += dO^T P and
//                        dK^T += Q^T dS (MFMA, A read from LDS with the transpose read, B
//                        straight from the S/dP accumulator registers).
//   fa_bwd_dq_kernel     one workgroup per (batch, head, 128 query rows), 32 rows per wave;
//                        Q^T and dO^T in VGPRs while 64-key tiles of K and V stream through LDS.
//                        Per tile: S^T = K Q^T and dP^T = V dO^T; P^T and dS^T elementwise;
//                        dQ^T += K^T dS^T.
// In every 32x32 accumulator a lane owns one column (a key in dkdv, a query row in dq) and 16
// rows 8(r/4) + 4hh + r%4; packing registers 8pc .. 8pc+7 of it gives the B operand of a
// 16-deep k-step whose k index e maps to row 16pc + 8(e/4) + 4hh + e%4, and the transpose read
// of the A operand uses the same map, so no shuffle is needed.
#pragma once

#include "fa_fwd_bf16.h"

namespace fa {

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;        // natural-log LSE of the forward pass [B, H, N]
    float* delta;            // workspace [B, H, N]: D_i = dO_i . O_i
    float* dq;
    float* dk;
    float* dv;
    const int32_t* seqlens;
    int B, H, N;
    float scale;             // multiplier of the raw dot products
    float scale_log2;        // scale * log2(e)
};

constexpr float kLog2e = 1.4426950408889634074f;

// XOR swizzle of the 16-byte chunk index within a tile row in LDS.  Rows are read both whole
// (16 bytes per lane) and with the 4 x 16 transpose read; the swizzle is a function of the row
// alone, so both read kinds address the same layout.
template <int D>
__device__ __forceinline__ int bwd_swz(int row) {
    return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

template <int D>
__device__ __forceinline__ int bwd_lds_off(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ bwd_swz<D>(row)) << 4);
}

// A operand of a 16-deep k-step from a row-major tile: lane (l32, hh) gets 8 consecutive
// columns 16c + 8hh .. of tile row r0 + l32.
template <int D>
__device__ __forceinline__ bf16x8 bwd_rowfrag(const unsigned char* tile, int r0, int l32, int hh, int c) {
    return *(const bf16x8*)(tile + bwd_lds_off<D>(r0 + l32, 2 * c + hh));
}

// A operand of the transposed tile (columns 32db .. 32db+31 as rows, tile rows 16pc .. +15 as
// the k index in the permuted order above), from two 4 x 16 transpose reads.
template <int D>
__device__ __forceinline__ bf16x8 bwd_trfrag(const unsigned char* tile, int l32, int hh, int pc, int db) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int vrow = 4 * hh + ((l32 & 15) >> 2);
    const int chunk = 4 * db + ((l32 & 16) >> 3) + ((l32 & 3) >> 1);
    const unsigned char* p0 = tile + (16 * pc + vrow) * (D * 2) + ((chunk ^ bwd_swz<D>(vrow)) << 4) + (l32 & 1) * 8;
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 8 * D * 2)));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Copies rows [g0, g0 + ROWS) of a [N, D] bf16 matrix into a swizzled LDS tile (rows past N
// are zero).  Split into fetch (global -> VGPRs, issued early) and stash (VGPRs -> LDS).
template <int D, int ROWS>
struct TileStage {
    static constexpr int CPR = D / 8;
    static constexpr int PER_THREAD = ROWS * CPR / 256;
    static_assert(PER_THREAD * 256 == ROWS * CPR, "tile must split evenly over 256 threads");
    bf16x8 r[PER_THREAD];
    __device__ __forceinline__ void fetch(const uint16_t* m, int g0, int N, int tid) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int id = i * 256 + tid, row = id / CPR, ch = id % CPR;
            const int g = g0 + row;
            r[i] = g < N ? *(const bf16x8*)(m + (int64_t)g * D + ch * 8) : bf16x8{};
        }
    }
    __device__ __forceinline__ void stash(unsigned char* tile, int tid) const {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int id = i * 256 + tid, row = id / CPR, ch = id % CPR;
            *(bf16x8*)(tile + bwd_lds_off<D>(row, ch)) = r[i];
        }
    }
};

// D_i = dO_i . O_i (float32 sum of bf16 products); D / 8 lanes per row.
template <int D>
__global__ void __launch_bounds__(256) fa_bwd_delta_kernel(BwdArgs a) {
    constexpr int LPR = D / 8;
    constexpr int RPB = 256 / LPR;
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    float s = 0.f;
    if (row < rows) {
        const bf16x8 x = *(const bf16x8*)((const uint16_t*)a.o + row * D + part * 8);
        const bf16x8 y = *(const bf16x8*)((const uint16_t*)a.dout + row * D + part * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf((float)x[e], (float)y[e], s);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (row < rows && part == 0) a.delta[row] = s;
}

template <int D, bool CAUSAL, bool PAD>
__global__ void __launch_bounds__(256, 1) fa_bwd_dkdv_kernel(BwdArgs a) {
    constexpr int BK = 128;        // keys per workgroup (32 per wave)
    constexpr int BQ = 32;         // query rows per tile
    constexpr int KC = D / 16;     // k-steps over d
    constexpr int NDB = D / 32;    // 32-wide blocks of d
    constexpr int TILEB = BQ * D * 2;
    __shared__ __attribute__((aligned(1024))) unsigned char qs[TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char dos[TILEB];
    __shared__ float lse2s[BQ];
    __shared__ float dls[BQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = a.N;
    // Work items in decreasing work order across all heads: under the causal mask key block kb
    // meets N/32 - 4kb query tiles, so every head's block 0 runs first, then every block 1 ...
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int k0 = (blockIdx.x / BH) * BK;
    const int b = bh / a.H;
    const int64_t base = (int64_t)bh * N * D;
    int Lk = N;
    if (PAD) {
        const int s = a.seqlens[b];
        Lk = s < 0 ? 0 : (s > N ? N : s);
    }
    const int key = k0 + wave * 32 + l32;    // this lane's key (column of every accumulator)

    // K^T and V^T as B operands ([k = d][n = key]): lane (key, hh) holds X[key][16c + 8hh ..]
    bf16x8 kt[KC], vt[KC];
    {
        const int kr = key < N ? key : 0;
        const uint16_t* kp = (const uint16_t*)a.k + base + (int64_t)kr * D + 8 * hh;
        const uint16_t* vp = (const uint16_t*)a.v + base + (int64_t)kr * D + 8 * hh;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            kt[c] = key < N ? *(const bf16x8*)(kp + 16 * c) : bf16x8{};
            vt[c] = key < N ? *(const bf16x8*)(vp + 16 * c) : bf16x8{};
        }
    }
    f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dkt[db] = dvt[db] = f32x16{};

    const int nt = (N + BQ - 1) / BQ;
    const int t0 = CAUSAL ? k0 / BQ : 0;        // earlier rows see none of these keys
    const bool live = k0 < Lk;                    // some key of this block is visible at all
    const uint16_t* qg = (const uint16_t*)a.q + base;
    const uint16_t* dog = (const uint16_t*)a.dout + base;
    const float* lse_g = a.lse + (int64_t)bh * N;
    const float* dl_g = a.delta + (int64_t)bh * N;
    TileStage<D, BQ> sq, sdo;
    float plse = 0.f, pdl = 0.f;
    auto fetch = [&](int t) __attribute__((always_inline)) {
        sq.fetch(qg, t * BQ, N, tid);
        sdo.fetch(dog, t * BQ, N, tid);
        if (tid < BQ) {
            const int g = t * BQ + tid;
            plse = g < N ? lse_g[g] * kLog2e : 0.f;
            pdl = g < N ? dl_g[g] : 0.f;
        }
    };
    if (live && t0 < nt) fetch(t0);
    for (int t = live ? t0 : nt; t < nt; ++t) {
        __syncthreads();                 // the previous tile is no longer read
        sq.stash(qs, tid);
        sdo.stash(dos, tid);
        if (tid < BQ) {
            lse2s[tid] = plse;
            dls[tid] = pdl;
        }
        __syncthreads();
        if (t + 1 < nt) fetch(t + 1);    // next tile's global loads overlap this tile's work

        // S = Q K^T and dP = dO V^T: lane (key, hh) holds rows 8(r/4) + 4hh + r%4 of the tile
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_rowfrag<D>(qs, 0, l32, hh, c), kt[c], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_rowfrag<D>(dos, 0, l32, hh, c), vt[c], dp, 0, 0, 0);
        }
        // P = exp(scale s - LSE) on visible (row, key) pairs, dS = P (dP - D)
        u32x4 ph[2], dsh[2];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            float p[2], ds[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int rr = 8 * ((r + u) >> 2) + 4 * hh + ((r + u) & 3);
                const int g = t * BQ + rr;
                const bool ok = g < N && key < Lk && (!CAUSAL || key <= g);
                const float e = fast_exp2(fmaf(s[r + u], a.scale_log2, -lse2s[rr]));
                p[u] = ok ? e : 0.f;
                ds[u] = p[u] * (dp[r + u] - dls[rr]);
            }
            ph[r / 8][(r % 8) / 2] = pack_bf16x2(p[0], p[1]);
            dsh[r / 8][(r % 8) / 2] = pack_bf16x2(ds[0], ds[1]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS (k runs over the tile's rows)
#pragma unroll
        for (int pc = 0; pc < 2; ++pc)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_trfrag<D>(dos, l32, hh, pc, db),
                                                                 __builtin_bit_cast(bf16x8, ph[pc]), dvt[db], 0, 0, 0);
                dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_trfrag<D>(qs, l32, hh, pc, db),
                                                                 __builtin_bit_cast(bf16x8, dsh[pc]), dkt[db], 0, 0, 0);
            }
    }
    // register r of block db is X^T[32db + 8(r/4) + 4hh + r%4][key]
    if (key < N) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = 32 * db + 8 * jj + 4 * hh;
                const int64_t off = base + (int64_t)key * D + d0;
                *(f32x4*)(a.dk + off) = f32x4{a.scale * dkt[db][4 * jj], a.scale * dkt[db][4 * jj + 1],
                                              a.scale * dkt[db][4 * jj + 2], a.scale * dkt[db][4 * jj + 3]};
                *(f32x4*)(a.dv + off) = f32x4{dvt[db][4 * jj], dvt[db][4 * jj + 1], dvt[db][4 * jj + 2],
                                              dvt[db][4 * jj + 3]};
            }
    }
}

template <int D, bool CAUSAL, bool PAD>
__global__ void __launch_bounds__(256, D == 128 ? 1 : 2) fa_bwd_dq_kernel(BwdArgs a) {
    constexpr int BM = 128;        // query rows per workgroup (32 per wave)
    constexpr int BN = 64;         // keys per tile
    constexpr int KC = D / 16;
    constexpr int NKB = BN / 32;
    constexpr int NDB = D / 32;
    constexpr int PC = BN / 16;
    constexpr int TILEB = BN * D * 2;
    __shared__ __attribute__((aligned(1024))) unsigned char ks[TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char vs[TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = a.N;
    // Work items in decreasing work order across all heads: under the causal mask query block
    // qb meets qb + 1 key blocks, so every head's last block runs first
    const int nqb = (N + BM - 1) / BM;
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int q0 = (CAUSAL ? nqb - 1 - blockIdx.x / BH : blockIdx.x / BH) * BM;
    const int b = bh / a.H;
    const int64_t base = (int64_t)bh * N * D;
    int Lk = N;
    if (PAD) {
        const int s = a.seqlens[b];
        Lk = s < 0 ? 0 : (s > N ? N : s);
    }
    const int row = q0 + wave * 32 + l32;    // this lane's query row (column of every accumulator)
    const bool row_ok = row < N;

    // Q^T and dO^T as B operands ([k = d][n = row])
    bf16x8 qt[KC], dot[KC];
    {
        const int rr = row_ok ? row : 0;
        const uint16_t* qp = (const uint16_t*)a.q + base + (int64_t)rr * D + 8 * hh;
        const uint16_t* dp = (const uint16_t*)a.dout + base + (int64_t)rr * D + 8 * hh;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            qt[c] = row_ok ? *(const bf16x8*)(qp + 16 * c) : bf16x8{};
            dot[c] = row_ok ? *(const bf16x8*)(dp + 16 * c) : bf16x8{};
        }
    }
    const float lse2 = row_ok ? a.lse[(int64_t)bh * N + row] * kLog2e : 0.f;
    const float dl = row_ok ? a.delta[(int64_t)bh * N + row] : 0.f;
    f32x16 dqt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqt[db] = f32x16{};

    int kv_end = Lk;
    if (CAUSAL) kv_end = kv_end < q0 + BM ? kv_end : q0 + BM;
    const int nj = (kv_end + BN - 1) / BN;
    const uint16_t* kg = (const uint16_t*)a.k + base;
    const uint16_t* vg = (const uint16_t*)a.v + base;
    TileStage<D, BN> sk, sv;
    if (nj > 0) {
        sk.fetch(kg, 0, N, tid);
        sv.fetch(vg, 0, N, tid);
    }
    for (int j = 0; j < nj; ++j) {
        __syncthreads();
        sk.stash(ks, tid);
        sv.stash(vs, tid);
        __syncthreads();
        if (j + 1 < nj) {
            sk.fetch(kg, (j + 1) * BN, N, tid);
            sv.fetch(vg, (j + 1) * BN, N, tid);
        }
        // S^T = K Q^T, dP^T = V dO^T: lane (row, hh) holds keys 32kb + 8(r/4) + 4hh + r%4
        f32x16 s[NKB], dp[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = dp[kb] = f32x16{};
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_rowfrag<D>(ks, 32 * kb, l32, hh, c), qt[c], s[kb], 0, 0, 0);
                dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_rowfrag<D>(vs, 32 * kb, l32, hh, c), dot[c], dp[kb], 0, 0, 0);
            }
        }
        // dS^T = P^T (dP^T - D) on visible pairs, packed as the B operand of dQ^T += K^T dS^T
        u32x4 dsh[PC];
#pragma unroll
        for (int f = 0; f < 16 * NKB; f += 2) {
            float ds[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int kb = (f + u) / 16, r = (f + u) % 16;
                const int key = j * BN + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                const bool ok = key < Lk && (!CAUSAL || key <= row);
                const float e = fast_exp2(fmaf(s[kb][r], a.scale_log2, -lse2));
                const float p = ok ? e : 0.f;
                ds[u] = p * (dp[kb][r] - dl);
            }
            dsh[f / 8][(f % 8) / 2] = pack_bf16x2(ds[0], ds[1]);
        }
#pragma unroll
        for (int pc = 0; pc < PC; ++pc)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                dqt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_trfrag<D>(ks, l32, hh, pc, db),
                                                                 __builtin_bit_cast(bf16x8, dsh[pc]), dqt[db], 0, 0, 0);
    }
    if (row_ok) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = 32 * db + 8 * jj + 4 * hh;
                *(f32x4*)(a.dq + base + (int64_t)row * D + d0) =
                    f32x4{a.scale * dqt[db][4 * jj], a.scale * dqt[db][4 * jj + 1], a.scale * dqt[db][4 * jj + 2],
                          a.scale * dqt[db][4 * jj + 3]};
            }
    }
}

}  // namespace fa
