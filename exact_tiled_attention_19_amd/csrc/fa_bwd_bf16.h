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
//                        wave's K^T and V^T stay in VGPRs while 64- or 32-row tiles of Q and dO
//                        stream global -> LDS directly (double-buffered, one barrier per tile).
//                        Per tile: S = Q K^T and dP = dO V^T (MFMA, A from LDS,
//                        B from VGPRs); P and dS elementwise; dV^T += dO^T P and
//                        dK^T += Q^T dS (MFMA, A read from LDS with the transpose read, B
//                        straight from the S/dP accumulator registers).
//   fa_bwd_dq_kernel     one workgroup per (batch, head, 128 query rows), 32 rows per wave;
//                        Q^T and dO^T in registers while 64-key tiles of K and V stream
//                        global -> LDS directly (double-buffered, no register staging).
//                        Per tile: S^T = K Q^T and dP^T = V dO^T; P^T and dS^T elementwise;
//                        dQ^T += K^T dS^T.
// In every 32x32 accumulator a lane owns one column (a key in dkdv, a query row in dq) and 16
// rows 8(r/4) + 4hh + r%4; packing registers 8pc .. 8pc+7 of it gives the B operand of a
// 16-deep k-step whose k index e maps to row 16pc + 8(e/4) + 4hh + e%4, and the transpose read
// of the A operand uses the same map, so no shuffle is needed.
#pragma once

#include "fa_fwd_bf16.h"
#include "fa_dropout.h"

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
    // dropout of the forward pass (kernels instantiated with dropout only; contract of
    // fa_fwd_dropout): dV = (P Z)^T dO, dP = Z (dO V^T), with Z = keep * keep_scale
    uint32_t drop_k0, drop_k1, drop_offset, drop_t;
    float drop_keep_scale;
};

constexpr float kLog2e = 1.4426950408889634074f;

// XOR swizzle of the 16-byte chunk index within a tile row in LDS.  Rows are read both whole
// (16 bytes per lane, 16 consecutive rows per pass of 16 lanes) and with the 4 x 16 transpose
// read (4 consecutive rows x 4 consecutive chunks per 32 lanes); the swizzle is a function of
// the row alone, so both read kinds address the same layout.  Bits 2-3 of the swizzle separate
// the 4 rows of a transpose read; the remaining bits make the 16 rows of a whole-row pass land
// on distinct banks (at d = 128 a row spans all 64 banks; at d = 64 two rows do, so only the 8
// rows of one parity must differ).
template <int D>
__device__ __forceinline__ int bwd_swz(int row) {
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
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
    const unsigned char* p1 = tile + (16 * pc + vrow + 8) * (D * 2) + ((chunk ^ bwd_swz<D>(vrow + 8)) << 4) + (l32 & 1) * 8;
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Waits until this wave's global -> LDS loads have completed (vmcnt(0)).
__device__ __forceinline__ void bwd_wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Two 4 x 16 transpose reads at LDS addresses p0 and p1, joined into one A operand.
__device__ __forceinline__ bf16x8 bwd_tr_pair(const unsigned char* p0, const unsigned char* p1) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// 16 bytes per lane from a buffer resource straight into LDS (lane i's bytes land at lds + 16 i).
// A plain device function: the builtin exists for the device only, and inside a template or
// lambda the host pass would drop the kernels that use it.
__device__ __forceinline__ void bwd_load_lds16(__amdgpu_buffer_rsrc_t rsrc, unsigned char* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Rows [g0, g0 + ROWS) of a [N, D] bf16 matrix straight from global memory into the swizzled
// LDS tile layout above, with buffer_load_dwordx4 ... lds (no register staging): each
// instruction fills 1 KiB of LDS in lane order, so lane lam of piece r writes physical chunk
// p = 64 r + lam (row p / CPR, chunk p % CPR) and fetches the logical chunk that the swizzle maps
// there.  The buffer's byte range ends with row N - 1, so rows past it read as zeros.  The
// loads complete asynchronously: wait for them (vmcnt) and a barrier before the tile is read.
template <int D, int ROWS, int NW>
struct TileDirect {
    static constexpr int CPR = D / 8;                     // 16-byte chunks per row
    static constexpr int LPW = ROWS * D * 2 / 1024 / NW;  // 1 KiB pieces per wave
    static_assert(LPW >= 1 && LPW * NW * 1024 == ROWS * D * 2, "tile must split into 1 KiB pieces per wave");
    uint32_t off[LPW];
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int p = (i * NW + wave) * 64 + lane;
            const int row = p / CPR, pch = p % CPR;
            off[i] = row * (D * 2) + ((pch ^ bwd_swz<D>(row)) << 4);
        }
    }
    __device__ __forceinline__ void load(unsigned char* tile, const uint16_t* m, int g0, int N, int wave) const {
        const int64_t left = (int64_t)(N - g0) * (D * 2);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(m + (int64_t)g0 * D), (short)0, left > 0 ? (int)(uint32_t)left : 0, 0x00020000);
#pragma unroll
        for (int i = 0; i < LPW; ++i) bwd_load_lds16(rs, tile + (i * NW + wave) * 1024, off[i]);
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

// Query rows per dK/dV tile.  d = 64: 32-row tiles keep two workgroups per CU.  d = 128 runs
// one workgroup per CU with 64-row tiles, two 32-row halves (without dropout each half's
// vector work rides on the other half's MFMAs).
template <int D>
constexpr int bwd_bq() { return D == 128 ? 64 : 32; }

template <int D, bool CAUSAL, bool PAD, bool DROP = false>
__global__ void __launch_bounds__(256, D == 64 ? 2 : 1) fa_bwd_dkdv_kernel(BwdArgs a) {
    constexpr int BK = 128;        // keys per workgroup (32 per wave)
    constexpr int BQ = bwd_bq<D>();  // query rows per tile, handled as 32-row halves
    constexpr int NH = BQ / 32;
    constexpr int KC = D / 16;     // k-steps over d
    constexpr int NDB = D / 32;    // 32-wide blocks of d
    constexpr int TILEB = BQ * D * 2;
    // double-buffered Q and dO tiles: tile t+1 is stored while tile t is read, one barrier a tile
    __shared__ __attribute__((aligned(1024))) unsigned char qs[2][TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char dos[2][TILEB];
    __shared__ __attribute__((aligned(16))) float lse2s[2][BQ];
    __shared__ __attribute__((aligned(16))) float dls[2][BQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = a.N;
    // Work items in decreasing work order across all heads: under the causal mask key block kb
    // meets (N - 128 kb) / BQ query tiles, so every head's block 0 runs first, then every block 1
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
    const int kw0 = k0 + wave * 32;          // first key of this wave
    const int key = kw0 + l32;               // this lane's key (column of every accumulator)

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
    const int t_begin = k0 < Lk ? t0 : nt;       // no visible key at all: nothing to accumulate
    const uint16_t* qg = (const uint16_t*)a.q + base;
    const uint16_t* dog = (const uint16_t*)a.dout + base;
    const float* lse_g = a.lse + (int64_t)bh * N;
    const float* dl_g = a.delta + (int64_t)bh * N;
    // Q and dO tiles go global -> LDS directly into the buffers that tile t-1 left (every wave
    // passed the barrier after reading them) while tile t is computed; the rows' LSE and D
    // values take a register round trip.  The buffers are numbered from t_begin, so the tile
    // loop below runs in pairs with literal parities and the LDS offsets are immediates.
    TileDirect<D, BQ, 4> ld;
    ld.init(wave, lane);
    float plse = 0.f, pdl = 0.f;
    auto fetch = [&](int t, int buf) __attribute__((always_inline)) {
        ld.load(qs[buf], qg, t * BQ, N, wave);
        ld.load(dos[buf], dog, t * BQ, N, wave);
        if (tid < BQ) {
            const int g = t * BQ + tid;
            plse = g < N ? lse_g[g] * kLog2e : 0.f;
            pdl = g < N ? dl_g[g] : 0.f;
        }
    };
    auto stash = [&](int buf) __attribute__((always_inline)) {
        if (tid < BQ) {
            lse2s[buf][tid] = plse;
            dls[buf][tid] = pdl;
        }
    };
    if (t_begin < nt) {
        fetch(t_begin, 0);
        bwd_wait_loads();
        stash(0);
    }
    __syncthreads();
    auto tile = [&](const int cur, int t) __attribute__((always_inline)) {
        if (t + 1 < nt) fetch(t + 1, cur ^ 1);   // global loads overlap this tile's work
        const unsigned char* qt_ = qs[cur];
        const unsigned char* dt_ = dos[cur];
        const float* ls = lse2s[cur];
        const float* dd = dls[cur];
        const int r0 = t * BQ;
        // the mask matters only where some row may not see some key of this wave (causal
        // diagonal, keys past the valid length or past N, rows past N)
        const bool masked = (CAUSAL && r0 < kw0 + 31) || kw0 + 32 > Lk || r0 + BQ > N;

        // S = Q K^T and dP = dO V^T per 32-row half: lane (key, hh) holds half rows
        // 8(r/4) + 4hh + r%4.  Computed inside each arm of the mask branch below, so that one
        // basic block holds the whole tile and half 0's vector work can overlap half 1's MFMAs.
        f32x16 s[NH], dp[NH];
        // Issue order (without dropout): one slot per k-step with its MFMAs, the LDS operands
        // read two slots ahead, slots kept apart by sched_barrier, so every read has four MFMAs
        // of time to return; hook(slot) places vector work beside them.  The d = 64 dropout
        // instantiations, whose mask bits take more registers, keep the compiler's own order
        // (the pinned one would spill there).
        auto sdp_h = [&](int h, auto hook) __attribute__((always_inline)) {
            s[h] = dp[h] = f32x16{};
            bf16x8 fq0 = bwd_rowfrag<D>(qt_, 32 * h, l32, hh, 0), fd0 = bwd_rowfrag<D>(dt_, 32 * h, l32, hh, 0);
            bf16x8 fq1 = bwd_rowfrag<D>(qt_, 32 * h, l32, hh, 1), fd1 = bwd_rowfrag<D>(dt_, 32 * h, l32, hh, 1);
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                bf16x8 fq2 = fq1, fd2 = fd1;
                if (c + 2 < KC) {
                    fq2 = bwd_rowfrag<D>(qt_, 32 * h, l32, hh, c + 2);
                    fd2 = bwd_rowfrag<D>(dt_, 32 * h, l32, hh, c + 2);
                }
                s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq0, kt[c], s[h], 0, 0, 0);
                dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fd0, vt[c], dp[h], 0, 0, 0);
                hook(c);
                fq0 = fq1;
                fd0 = fd1;
                fq1 = fq2;
                fd1 = fd2;
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto prod_h = [&](int h, const u32x4 (&ph)[2], const u32x4 (&dsh)[2], auto hook) __attribute__((always_inline)) {
            constexpr int NP = 2 * NDB;
            bf16x8 fd0 = bwd_trfrag<D>(dt_, l32, hh, 2 * h, 0), fq0 = bwd_trfrag<D>(qt_, l32, hh, 2 * h, 0);
            bf16x8 fd1 = bwd_trfrag<D>(dt_, l32, hh, 2 * h + 1 / NDB, 1 % NDB);
            bf16x8 fq1 = bwd_trfrag<D>(qt_, l32, hh, 2 * h + 1 / NDB, 1 % NDB);
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int pc = i / NDB, db = i % NDB;
                bf16x8 fd2 = fd1, fq2 = fq1;
                if (i + 2 < NP) {
                    fd2 = bwd_trfrag<D>(dt_, l32, hh, 2 * h + (i + 2) / NDB, (i + 2) % NDB);
                    fq2 = bwd_trfrag<D>(qt_, l32, hh, 2 * h + (i + 2) / NDB, (i + 2) % NDB);
                }
                dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fd0, __builtin_bit_cast(bf16x8, ph[pc]), dvt[db], 0, 0, 0);
                dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq0, __builtin_bit_cast(bf16x8, dsh[pc]), dkt[db], 0, 0, 0);
                hook(i);
                fd0 = fd1;
                fq0 = fq1;
                fd1 = fd2;
                fq1 = fq2;
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto sdp = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                if constexpr (DROP && D == 64) {
                    s[h] = dp[h] = f32x16{};
#pragma unroll
                    for (int c = 0; c < KC; ++c) {
                        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_rowfrag<D>(qt_, 32 * h, l32, hh, c), kt[c], s[h], 0, 0, 0);
                        dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_rowfrag<D>(dt_, 32 * h, l32, hh, c), vt[c], dp[h], 0, 0, 0);
                    }
                } else {
                    sdp_h(h, [](int) {});
                }
            }
        };
        // P = exp(scale s - LSE) on visible pairs, dS = P (dP - D); then dV^T += dO^T P and
        // dK^T += Q^T dS over the half's rows.  Half 1's products overlap half 0's vector work.
        auto half = [&](int h, auto masked_c) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_c)::value;
            u32x4 ph[2], dsh[2];
            uint32_t kbits = 0;   // dropout: bit 4 (r / 4) + r % 4 set iff element r is kept
            if constexpr (DROP)
                kbits = dropout_bits_kmajor(key, r0 + 32 * h, hh, bh, a.drop_offset, a.drop_k0, a.drop_k1, a.drop_t);
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                const int rr = 32 * h + 8 * (r >> 2) + 4 * hh;       // rows rr .. rr+3
                const f32x4 l4 = *(const f32x4*)(ls + rr);
                const f32x4 d4 = *(const f32x4*)(dd + rr);
                float p[4], ds[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float e = fast_exp2(fmaf(s[h][r + u], a.scale_log2, -l4[u]));
                    if constexpr (MASKED) {
                        const int g = r0 + rr + u;
                        const bool ok = g < N && key < Lk && (!CAUSAL || key <= g);
                        e = ok ? e : 0.f;
                    }
                    if constexpr (DROP) {
                        // dV takes P Z (Z's scale applied to dV at the end), dS = P (Z dP~ - D)
                        const bool keep = (kbits >> (r + u)) & 1u;
                        p[u] = keep ? e : 0.f;
                        ds[u] = e * ((keep ? a.drop_keep_scale * dp[h][r + u] : 0.f) - d4[u]);
                    } else {
                        p[u] = e;
                        ds[u] = e * (dp[h][r + u] - d4[u]);
                    }
                }
                ph[r / 8][(r % 8) / 2] = pack_bf16x2(p[0], p[1]);
                ph[r / 8][(r % 8) / 2 + 1] = pack_bf16x2(p[2], p[3]);
                dsh[r / 8][(r % 8) / 2] = pack_bf16x2(ds[0], ds[1]);
                dsh[r / 8][(r % 8) / 2 + 1] = pack_bf16x2(ds[2], ds[3]);
            }
            if constexpr (DROP && D == 64) {
#pragma unroll
                for (int pc = 0; pc < 2; ++pc)
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_trfrag<D>(dt_, l32, hh, 2 * h + pc, db),
                                                                         __builtin_bit_cast(bf16x8, ph[pc]), dvt[db], 0, 0, 0);
                        dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_trfrag<D>(qt_, l32, hh, 2 * h + pc, db),
                                                                         __builtin_bit_cast(bf16x8, dsh[pc]), dkt[db], 0, 0, 0);
                    }
            } else {
                prod_h(h, ph, dsh, [](int) {});
            }
        };
        // Two halves without dropout: the tile as one sequence of slots in which each half's
        // vector work rides on the other half's MFMAs -- half 0's P and dS on the S/dP products
        // of half 1, half 1's on the dV/dK products of half 0 -- instead of running between them.
        // P and dS of rows 4rq .. 4rq+3 of half h's 32-row block (lane rows 8rq + 4hh ..)
        auto pds = [&](int h, int rq, auto masked_c, u32x4 (&ph)[2], u32x4 (&dsh)[2]) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_c)::value;
            const int r = 4 * rq;
            const int rr = 32 * h + 8 * rq + 4 * hh;
            const f32x4 l4 = *(const f32x4*)(ls + rr);
            const f32x4 d4 = *(const f32x4*)(dd + rr);
            float p[4], ds[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float e = fast_exp2(fmaf(s[h][r + u], a.scale_log2, -l4[u]));
                if constexpr (MASKED) {
                    const int g = r0 + rr + u;
                    const bool ok = g < N && key < Lk && (!CAUSAL || key <= g);
                    e = ok ? e : 0.f;
                }
                p[u] = e;
                ds[u] = e * (dp[h][r + u] - d4[u]);
            }
            ph[r / 8][(r % 8) / 2] = pack_bf16x2(p[0], p[1]);
            ph[r / 8][(r % 8) / 2 + 1] = pack_bf16x2(p[2], p[3]);
            dsh[r / 8][(r % 8) / 2] = pack_bf16x2(ds[0], ds[1]);
            dsh[r / 8][(r % 8) / 2 + 1] = pack_bf16x2(ds[2], ds[3]);
        };
        auto piped = [&](auto masked_c) __attribute__((always_inline)) {
            u32x4 ph0[2], dsh0[2], ph1[2], dsh1[2];
            sdp_h(0, [&](int) {});
            sdp_h(1, [&](int c) { if (c & 1) pds(0, c >> 1, masked_c, ph0, dsh0); });
            prod_h(0, ph0, dsh0, [&](int i) { if (i & 1) pds(1, i >> 1, masked_c, ph1, dsh1); });
            prod_h(1, ph1, dsh1, [&](int) {});
        };
        constexpr bool PIPED = !DROP && NH == 2 && KC == 8 && NDB == 4;
        if constexpr (PIPED) {
            if (masked) piped(std::true_type{});
            else piped(std::false_type{});
        } else if (masked) {
            sdp();
#pragma unroll
            for (int h = 0; h < NH; ++h) half(h, std::true_type{});
        } else {
            sdp();
#pragma unroll
            for (int h = 0; h < NH; ++h) half(h, std::false_type{});
        }
        bwd_wait_loads();                        // tile t+1 is in LDS
        if (t + 1 < nt) stash(cur ^ 1);
        __syncthreads();
    };
    int t = t_begin;
    for (; t + 2 <= nt; t += 2) {
        tile(0, t);
        tile(1, t + 1);
    }
    if (t < nt) tile(0, t);
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
                const float vs = DROP ? a.drop_keep_scale : 1.f;
                *(f32x4*)(a.dv + off) = f32x4{vs * dvt[db][4 * jj], vs * dvt[db][4 * jj + 1], vs * dvt[db][4 * jj + 2],
                                              vs * dvt[db][4 * jj + 3]};
            }
    }
}

template <int D, bool CAUSAL, bool PAD, bool DROP = false>
__global__ void __launch_bounds__(256, D == 128 ? 1 : 2) fa_bwd_dq_kernel(BwdArgs a) {
    constexpr int BM = 128;        // query rows per workgroup (32 per wave)
    constexpr int BN = 64;         // keys per tile
    constexpr int KC = D / 16;
    constexpr int NKB = BN / 32;
    constexpr int NDB = D / 32;
    constexpr int TILEB = BN * D * 2;
    __shared__ __attribute__((aligned(1024))) unsigned char ks[2][TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char vs[2][TILEB];

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
    const int qw0 = q0 + wave * 32;          // first query row of this wave
    const int row = qw0 + l32;               // this lane's query row (column of every accumulator)
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
    // K and V tiles go straight to LDS; tile j+1 is loaded into the buffers that tile j-1 left
    // (every wave passed the barrier after reading them) while tile j is computed
    TileDirect<D, BN, 4> ld;
    ld.init(wave, lane);
    // per-lane LDS byte offsets (the tile and block offsets are added as constants): whole-row
    // operand of k-step c (row l32, chunk 2c + hh), and the two transpose reads of block db
    // (rows vrow and vrow + 8 of the 16-row step, bwd_trfrag's addressing)
    constexpr int ROWB = D * 2;
    int roff[KC], toff0[NDB], toff1[NDB];
#pragma unroll
    for (int c = 0; c < KC; ++c) roff[c] = bwd_lds_off<D>(l32, 2 * c + hh);
    {
        const int vrow = 4 * hh + ((l32 & 15) >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int chunk = 4 * db + ((l32 & 16) >> 3) + ((l32 & 3) >> 1);
            toff0[db] = vrow * ROWB + ((chunk ^ bwd_swz<D>(vrow)) << 4) + (l32 & 1) * 8;
            toff1[db] = (vrow + 8) * ROWB + ((chunk ^ bwd_swz<D>(vrow + 8)) << 4) + (l32 & 1) * 8;
        }
    }
    auto rfrag = [&](const unsigned char* t, int kb, int c) __attribute__((always_inline)) -> bf16x8 {
        return *(const bf16x8*)(t + 32 * kb * ROWB + roff[c]);
    };
    auto tfrag = [&](const unsigned char* t, int pc, int db) __attribute__((always_inline)) -> bf16x8 {
        return bwd_tr_pair(t + 16 * pc * ROWB + toff0[db], t + 16 * pc * ROWB + toff1[db]);
    };
    if (nj > 0) {
        ld.load(ks[0], kg, 0, N, wave);
        ld.load(vs[0], vg, 0, N, wave);
    }
    bwd_wait_loads();
    __syncthreads();
    // One tile; the loop below runs tiles in pairs with literal buffer parities, so after inlining
    // every LDS address is a per-lane register plus an immediate offset.
    auto tile = [&](const int cur, int j) __attribute__((always_inline)) {
        if (j + 1 < nj) {
            ld.load(ks[cur ^ 1], kg, (j + 1) * BN, N, wave);
            ld.load(vs[cur ^ 1], vg, (j + 1) * BN, N, wave);
        }
        const unsigned char* kt_ = ks[cur];
        const unsigned char* vt_ = vs[cur];
        const int j0 = j * BN;
        // the mask matters only where some key of the tile lies past a row of this wave (causal
        // diagonal) or past the valid length (and past N)
        const bool masked = (CAUSAL && j0 + BN - 1 > qw0) || j0 + BN > Lk;
        // S^T = K Q^T, dP^T = V dO^T per 32-key block: lane (row, hh) holds keys
        // 32kb + 8(r/4) + 4hh + r%4 (inside each arm of the mask branch, as in the dK/dV kernel).
        // One 32-key block at a time (its S^T, dP^T, dS^T and dQ^T products), so that only one
        // block's scores are live.  Issue order: one slot per k-step with its two MFMAs, the LDS
        // operands read two slots ahead, slots kept apart by sched_barrier, so at most three
        // slots' fragments are live and every read has two MFMAs of time to return.
        f32x16 s[NKB], dp[NKB];
        auto sdp_k = [&](int kb, auto hook) __attribute__((always_inline)) {
            s[kb] = dp[kb] = f32x16{};
            bf16x8 kf0 = rfrag(kt_, kb, 0), vf0 = rfrag(vt_, kb, 0);
            bf16x8 kf1 = rfrag(kt_, kb, 1), vf1 = rfrag(vt_, kb, 1);
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                bf16x8 kf2 = kf1, vf2 = vf1;
                if (c + 2 < KC) {
                    kf2 = rfrag(kt_, kb, c + 2);
                    vf2 = rfrag(vt_, kb, c + 2);
                }
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qt[c], s[kb], 0, 0, 0);
                dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf0, dot[c], dp[kb], 0, 0, 0);
                hook(c);
                kf0 = kf1;
                kf1 = kf2;
                vf0 = vf1;
                vf1 = vf2;
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto prod_k = [&](int kb, const u32x4 (&dsh)[2], auto hook) __attribute__((always_inline)) {
            constexpr int NP = 2 * NDB;
            bf16x8 f0 = tfrag(kt_, 2 * kb, 0);
            bf16x8 f1 = tfrag(kt_, 2 * kb + 1 / NDB, 1 % NDB);
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int pc = i / NDB, db = i % NDB;
                bf16x8 f2 = f1;
                if (i + 2 < NP) f2 = tfrag(kt_, 2 * kb + (i + 2) / NDB, (i + 2) % NDB);
                dqt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0, __builtin_bit_cast(bf16x8, dsh[pc]), dqt[db], 0, 0, 0);
                hook(i);
                f0 = f1;
                f1 = f2;
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto sdp = [&](int kb) __attribute__((always_inline)) { sdp_k(kb, [](int) {}); };
        // dS^T = P^T (dP^T - D) on visible pairs, packed as the B operand of dQ^T += K^T dS^T
        auto block = [&](int kb, auto masked_c) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_c)::value;
            u32x4 dsh[2];
            uint32_t dw[4];   // dropout words of this 32-key block (forward layout)
            if constexpr (DROP) dropout_words_fwd(dw, j0, kb, row, hh, bh, a.drop_offset, a.drop_k0, a.drop_k1);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float ds[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float e = fast_exp2(fmaf(s[kb][r + u], a.scale_log2, -lse2));
                    if constexpr (MASKED) {
                        const int key = j0 + 32 * kb + 8 * ((r + u) >> 2) + 4 * hh + ((r + u) & 3);
                        const bool ok = key < Lk && (!CAUSAL || key <= row);
                        e = ok ? e : 0.f;
                    }
                    if constexpr (DROP) {
                        const bool keep = drop_keep(dw[(r + u) >> 2], (r + u) & 3, a.drop_t);
                        ds[u] = e * ((keep ? a.drop_keep_scale * dp[kb][r + u] : 0.f) - dl);
                    } else {
                        ds[u] = e * (dp[kb][r + u] - dl);
                    }
                }
                dsh[r / 8][(r % 8) / 2] = pack_bf16x2(ds[0], ds[1]);
            }
            prod_k(kb, dsh, [](int) {});
        };
        // dS^T of keys 8(it/4) + 4hh + (2it)%8 .. +1 of block kb (registers 2it, 2it + 1)
        auto ds_pair = [&](int kb, int it, auto masked_c, u32x4 (&dsh)[2]) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_c)::value;
            const int r = 2 * it;
            float ds[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float e = fast_exp2(fmaf(s[kb][r + u], a.scale_log2, -lse2));
                if constexpr (MASKED) {
                    const int key = j0 + 32 * kb + 8 * ((r + u) >> 2) + 4 * hh + ((r + u) & 3);
                    const bool ok = key < Lk && (!CAUSAL || key <= row);
                    e = ok ? e : 0.f;
                }
                ds[u] = e * (dp[kb][r + u] - dl);
            }
            dsh[r / 8][(r % 8) / 2] = pack_bf16x2(ds[0], ds[1]);
        };
        // Without dropout the two key blocks run as one sequence of slots in which each block's
        // dS^T work rides on the other block's MFMAs: block 0's on the S^T/dP^T products of
        // block 1, block 1's on the dQ^T products of block 0.
        auto piped = [&](auto masked_c) __attribute__((always_inline)) {
            constexpr int NP = 2 * NDB;
            u32x4 dsh0[2], dsh1[2];
            sdp_k(0, [&](int) {});
            sdp_k(1, [&](int c) {
#pragma unroll
                for (int it = c * 8 / KC; it < (c + 1) * 8 / KC; ++it) ds_pair(0, it, masked_c, dsh0);
            });
            prod_k(0, dsh0, [&](int i) {
#pragma unroll
                for (int it = i * 8 / NP; it < (i + 1) * 8 / NP; ++it) ds_pair(1, it, masked_c, dsh1);
            });
            prod_k(1, dsh1, [&](int) {});
        };
        if constexpr (!DROP && NKB == 2) {
            if (masked) piped(std::true_type{});
            else piped(std::false_type{});
        } else if (masked) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                sdp(kb);
                block(kb, std::true_type{});
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                sdp(kb);
                block(kb, std::false_type{});
            }
        }
        bwd_wait_loads();   // tile j+1 is in LDS
        __syncthreads();
    };
    int j = 0;
    for (; j + 2 <= nj; j += 2) {
        tile(0, j);
        tile(1, j + 1);
    }
    if (j < nj) tile(0, j);
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
