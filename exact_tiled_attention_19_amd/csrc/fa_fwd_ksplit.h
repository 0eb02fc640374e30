// Key-split forward for launches too small to fill the chip (fewer work items than compute
// units, e.g. one head of a few thousand tokens).
//
// The NW waves of a workgroup (eight at d = 64, four at d = 128) share one 32-row query block
// and divide its 64-key tiles among themselves: wave w takes tiles w, w+NW, w+2NW, ...  Each
// wave keeps the running maximum, sum and unnormalised accumulator of the online update
// ("FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical Stability",
// section "How can softmax be computed across tiles?") over its own keys, and at the end the NW
// states are merged with the same rescaling: m = max_w m_w, l = sum_w 2^(m_w - m) l_w,
// O = sum_w 2^(m_w - m) acc_w / l.  The chain of tiles one wave walks is about NW times
// shorter than in the main kernel, and that chain is what bounds a launch with fewer
// workgroups than compute units.
//
// Each wave stages its own K and V tiles in its own LDS region (global -> registers -> LDS,
// the next tile's loads in flight while the current one is computed), so the tile loop needs
// no workgroup barrier.  Every workgroup reads all of its head's keys and values, and the
// per-CU load path and LDS traffic bound this kernel more than its MFMAs do.  The
// probabilities enter the value product as two bf16 terms (P_hi + P_lo) with a float32 output
// and in masked tiles, which hold every key of a row that sees fewer than one tile of keys;
// otherwise as one bf16 term, as in the main kernel.
//
// F8: FP8 E4M3 inputs with per-tensor descales, as in the pipelined FP8 kernel: S on the 8-bit
// MFMA with Q and K fragments taking the same byte -> dimension assignment, V widened to bf16
// (exactly) as it is written to LDS, the value descale applied to the output.
#pragma once

#include <type_traits>

#include "fa_fwd_bf16_pipe.h"

namespace fa {

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int D, bool CAUSAL, bool PAD, bool OUT_F32, int NW = 8, bool F8 = false>
__global__ void __launch_bounds__(64 * NW, 1) fa_fwd_bf16_ksplit_kernel(FwdArgs a) {
    // NW waves; each walks every NW-th key tile
    constexpr int BM = 32;                     // query rows per workgroup (one MFMA block)
    constexpr int BN = 64;                     // keys per tile
    constexpr int RPW = 16 / NW;               // accumulator registers per block each wave finishes
    constexpr int ESZ = F8 ? 1 : 2;            // bytes per input element
    constexpr int KC = F8 ? D / 64 : D / 16;   // k-steps of the S MFMA
    constexpr int NKB = BN / 32;               // 32-key blocks per tile
    constexpr int NDB = D / 32;                // 32-wide output blocks
    constexpr int PC = BN / 16;                // k-steps of the PV MFMA
    constexpr int KROWB = D * ESZ + 16;        // K row stride in LDS (bytes): 16-byte pad
    // V row stride in LDS (bf16 elements): a 64-byte pad, 32 bytes where eight waves' tiles
    // would not fit the 160 KiB otherwise
    constexpr int VSTR = D + ((NW == 8 && D * ESZ == 128) ? 16 : 32);
    constexpr int WBUFB = BN * KROWB + BN * VSTR * 2;   // bytes of one wave's K and V tiles
    constexpr int CPR = D * ESZ / 16;          // 16-byte input chunks per row
    constexpr int LDC = BN * CPR / 64;         // chunks per lane per tensor per tile
    constexpr int MACC = 64 * 16 * NDB;        // floats of one wave's accumulator
    constexpr int MERGEB = (2 * NW * 32 + NW * MACC) * 4;   // bytes of the merge state
    constexpr int SMEMB = NW * WBUFB > MERGEB ? NW * WBUFB : MERGEB;
    using KFrag = std::conditional_t<F8, i32x8, bf16x8>;
    static_assert(LDC * 64 == BN * CPR, "a tile must split evenly over the 64 lanes");
    static_assert((NW == 4 || NW == 8) && RPW * NW == 16, "each wave finishes whole register groups");
    static_assert(KROWB % 16 == 0 && WBUFB % 16 == 0, "16-byte LDS accesses stay aligned");
    static_assert(SMEMB <= 160 * 1024, "the buffers fit the LDS");

    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEMB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const TileCoord tc = tile_of(xcd_remap(blockIdx.x, a.total_wgs), a.n_qtiles, CAUSAL);
    const int b = tc.bh / a.H;
    const int N = a.N;
    const int q0 = tc.qt * BM;
    const int qrow = q0 + l32;                 // the query row of this lane (every wave)
    const int64_t base = (int64_t)tc.bh * N * D;

    int Lk = N;
    if (PAD) {
        const int s = a.seqlens[b];
        Lk = s < 0 ? 0 : (s > N ? N : s);
    }
    if (Lk == 0) {  // every key masked: O = 0, LSE = -inf (written by wave 0)
        if (wave == 0 && qrow < N) {
            if (hh == 0 && a.lse) a.lse[(int64_t)tc.bh * N + qrow] = kNegInf;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = 32 * db + 8 * j + 4 * hh;
                    if (OUT_F32) *(f32x4*)((float*)a.o + base + (int64_t)qrow * D + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
                    else *(u32x2*)((uint16_t*)a.o + base + (int64_t)qrow * D + d0) = u32x2{0u, 0u};
                }
        }
        return;
    }

    int kv_end = Lk;
    if (CAUSAL) kv_end = kv_end < q0 + BM ? kv_end : q0 + BM;
    const int n_tiles = (kv_end + BN - 1) / BN;   // >= 1: key 0 is visible to every row

    // Q^T operand: bf16 Q[qrow][16c + 8hh .. +8]; 8-bit: bytes 64c + 32hh .. +32 of the row (the
    // K fragments below take the same bytes of their rows)
    KFrag qf[KC];
    {
        const unsigned char* qp = (const unsigned char*)a.q + (base + (int64_t)(qrow < N ? qrow : N - 1) * D) * ESZ;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            if constexpr (F8)
                qf[c] = __builtin_bit_cast(i32x8, u32x8_of(*(const u32x4*)(qp + 64 * c + 32 * hh),
                                                           *(const u32x4*)(qp + 64 * c + 32 * hh + 16)));
            else
                qf[c] = *(const bf16x8*)(qp + 32 * c + 16 * hh);
            if (qrow >= N) qf[c] = KFrag{};
        }
    }

    unsigned char* const ks = smem + wave * WBUFB;              // this wave's K tile (bytes)
    uint16_t* const vs = (uint16_t*)(ks + BN * KROWB);          // and V tile (bf16)
    const unsigned char* const kg = (const unsigned char*)a.k + base * ESZ;
    const unsigned char* const vg = (const unsigned char*)a.v + base * ESZ;
    // chunk ci = lane + 64 i of a tile: row ci / CPR, column chunk ci % CPR.  The loads go through
    // buffer resources that start at the tile and end at key N, so rows past N read as zeros
    // (they are masked) and the per-tile address arithmetic is scalar.
    int goff[LDC];
#pragma unroll
    for (int i = 0; i < LDC; ++i) {
        const int ci = lane + 64 * i;
        goff[i] = (ci / CPR) * D * ESZ + (ci % CPR) * 16;
    }
    u32x4 kr[LDC], vr[LDC];   // the next tile on its way to LDS
    auto gload = [&](int tile) __attribute__((always_inline)) {
        const int64_t toff = static_cast<int64_t>(tile) * BN * D * ESZ;
        const int rec = (N - tile * BN) * D * ESZ;
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(kg + toff), (short)0, rec, 0x00020000);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(vg + toff), (short)0, rec, 0x00020000);
#pragma unroll
        for (int i = 0; i < LDC; ++i) {
            kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, goff[i], 0, 0));
            vr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, goff[i], 0, 0));
        }
    };
    auto swrite = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LDC; ++i) {
            const int ci = lane + 64 * i;
            const int row = ci / CPR;
            *(u32x4*)(ks + row * KROWB + (ci % CPR) * 16) = kr[i];
            if constexpr (F8) {   // 16 codes = dimensions 16 (ci % CPR) .. +16, widened to bf16
                const u32x2 w0 = e4m3x4_to_bf16(vr[i][0]), w1 = e4m3x4_to_bf16(vr[i][1]);
                const u32x2 w2 = e4m3x4_to_bf16(vr[i][2]), w3 = e4m3x4_to_bf16(vr[i][3]);
                *(u32x4*)(vs + row * VSTR + (ci % CPR) * 16) = u32x4{w0[0], w0[1], w1[0], w1[1]};
                *(u32x4*)(vs + row * VSTR + (ci % CPR) * 16 + 8) = u32x4{w2[0], w2[1], w3[0], w3[1]};
            } else {
                *(u32x4*)(vs + row * VSTR + (ci % CPR) * 8) = vr[i];
            }
        }
        // the wave's other lanes read what this lane wrote: wait for the writes to complete
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
    };
    // V^T operand of key chunk pc and output block db by LDS transpose reads: lane (d = 32db +
    // l32, hh) receives V[16pc + 8(e/4) + 4hh + e%4][d] for e = 0..7, the key order in which the
    // S^T accumulator holds this lane's probabilities
    auto vt_frag = [&](int pc, int db) __attribute__((always_inline)) -> bf16x8 {
        const int row = 16 * pc + 4 * hh + ((l32 & 15) >> 2);
        const int col = 32 * db + (l32 & 16) + 4 * (l32 & 3);
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + row * VSTR + col)));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + (row + 8) * VSTR + col)));
        return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };

    float m_run = kNegInf;   // running maximum of scale*log2(e)*s over this wave's visible keys
    float l_run = 0.f;       // this lane half's running sum of 2^(.. - m_run)
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    // wave w takes tiles w, w + NW, w + 2 NW, ...: R of them
    const int n_rounds = (n_tiles + NW - 1) / NW;
    const int R = wave < n_tiles - (n_rounds - 1) * NW ? n_rounds : n_rounds - 1;
    auto tile_at = [&](int j) __attribute__((always_inline)) { return j * NW + wave; };
    // one key tile: S, mask, online update, O += P V (its K and V are in this wave's LDS
    // buffer).  MASKED: the tile holds a key past Lk or, under the causal mask, past a row.
    auto tile_step = [&](int t, auto masked_c) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_c)::value;
        const int kv0 = t * BN;
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const unsigned char* kp = ks + (32 * kb + l32) * KROWB;
                KFrag kf;
                if constexpr (F8)
                    kf = __builtin_bit_cast(i32x8, u32x8_of(*(const u32x4*)(kp + 64 * c + 32 * hh),
                                                            *(const u32x4*)(kp + 64 * c + 32 * hh + 16)));
                else
                    kf = *(const bf16x8*)(kp + 32 * c + 16 * hh);
                s[kb] = mfma_s(kf, qf[c], s[kb]);
            }
        }
        // accumulator register r of block kb holds key kv0 + 32kb + 8(r/4) + 4hh + r%4
        if constexpr (MASKED) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const bool ok = key < Lk && (!CAUSAL || key <= qrow);
                    s[kb][r] = ok ? s[kb][r] : kNegInf;
                }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = xor32_max(mx);
        // the scale is positive, so the largest score gives the largest scaled logit; a tile
        // without masked keys has a finite maximum
        const float m_tile = (MASKED && mx == kNegInf) ? kNegInf : mx * a.scale_log2;
        const float m_new = fmaxf(m_run, m_tile);
        const float m_use = (MASKED && m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(fmaf(s[kb][r], a.scale_log2, -m_use));
                if constexpr (MASKED) p = s[kb][r] == kNegInf ? 0.f : p;   // exact zeros, also when scale == 0
                s[kb][r] = p;
                rs += p;
            }
        l_run = alpha * l_run + rs;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
        // O^T += V^T P^T; key chunk pc = registers 8(pc % 2) .. +7 of block pc / 2
        auto pv = [&](auto split_c) __attribute__((always_inline)) {
            constexpr bool SPLIT = decltype(split_c)::value;
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) {
                const int kb = pc >> 1;
                const int r0 = 8 * (pc & 1);
                u32x4 ph, pl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ph[e] = pack_bf16x2(s[kb][r0 + 2 * e], s[kb][r0 + 2 * e + 1]);
                    if constexpr (SPLIT)
                        pl[e] = pack_bf16x2(s[kb][r0 + 2 * e] - bf16_lo_to_f32(ph[e]),
                                            s[kb][r0 + 2 * e + 1] - bf16_hi_to_f32(ph[e]));
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 vf = vt_frag(pc, db);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, ph), acc[db], 0, 0, 0);
                    if constexpr (SPLIT)
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, pl), acc[db], 0, 0, 0);
                }
            }
        };
        pv(std::integral_constant<bool, OUT_F32 || MASKED>{});
    };
    // Step i computes tile i from LDS while the loads of tile i+1 are in flight, then moves
    // tile i+1 from registers to LDS
    if (R > 0) {
        gload(tile_at(0));
        swrite();
        for (int i = 0; i < R; ++i) {
            const bool more = i + 1 < R;
            if (more) gload(tile_at(i + 1));
            const int t = tile_at(i);
            if (t * BN + BN > Lk || (CAUSAL && t * BN + BN - 1 > q0)) tile_step(t, std::true_type{});
            else tile_step(t, std::false_type{});
            if (more) swrite();   // this tile's reads have all returned (their MFMAs used them)
        }
    }

    // merge.  LDS layout (floats): maxima [NW][32], sums [NW][32], accumulators
    // [NW][4 NDB][64][4]: register group j (registers 4j .. 4j+3) of block db of wave v at
    // [v][4 db + j][lane], so the 64 lanes of one access touch consecutive 16-byte slots.
    __syncthreads();   // every wave is done with its tile buffers
    float* const ms = reinterpret_cast<float*>(smem);
    float* const ls = ms + NW * 32;
    float* const as = ls + NW * 32;
    const float l_tot = xor32_sum(l_run);
    if (hh == 0) {
        ms[wave * 32 + l32] = m_run;
        ls[wave * 32 + l32] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *(f32x4*)(as + ((wave * 4 * NDB + 4 * db + j) * 64 + lane) * 4) =
                f32x4{acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]};
    __syncthreads();
    // wave w finishes accumulator registers RPW w .. RPW w + RPW - 1 of every block: register r
    // holds output column 32db + 8(r/4) + 4hh + r%4 of row qrow, so these are RPW adjacent
    // columns
    float m = kNegInf;
#pragma unroll
    for (int v = 0; v < NW; ++v) m = fmaxf(m, ms[v * 32 + l32]);
    float sc[NW];
    float l = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const float mv = ms[v * 32 + l32];
        sc[v] = mv == kNegInf ? 0.f : fast_exp2(mv - m);   // a wave without keys adds nothing
        l += sc[v] * ls[v * 32 + l32];
    }
    if (qrow >= N) return;
    if (wave == 0 && hh == 0 && a.lse) a.lse[(int64_t)tc.bh * N + qrow] = (m + __log2f(l)) * kLn2;
    const float inv_l = (F8 ? a.v_descale : 1.0f) / l;   // 8-bit inputs: V's descale
    const int r0 = RPW * wave;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        float o[RPW];
#pragma unroll
        for (int u = 0; u < RPW; ++u) o[u] = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const float* src = as + ((v * 4 * NDB + 4 * db + r0 / 4) * 64 + lane) * 4 + r0 % 4;
#pragma unroll
            for (int u = 0; u < RPW; ++u) o[u] += sc[v] * src[u];
        }
        const int d0 = 32 * db + 8 * (r0 / 4) + 4 * hh + r0 % 4;
        if constexpr (RPW == 4) {
            if (OUT_F32) *(f32x4*)((float*)a.o + base + (int64_t)qrow * D + d0) = f32x4{o[0] * inv_l, o[1] * inv_l, o[2] * inv_l, o[3] * inv_l};
            else *(u32x2*)((uint16_t*)a.o + base + (int64_t)qrow * D + d0) = u32x2{pack_bf16x2(o[0] * inv_l, o[1] * inv_l), pack_bf16x2(o[2] * inv_l, o[3] * inv_l)};
        } else {
            if (OUT_F32) *(f32x2*)((float*)a.o + base + (int64_t)qrow * D + d0) = f32x2{o[0] * inv_l, o[1] * inv_l};
            else *(uint32_t*)((uint16_t*)a.o + base + (int64_t)qrow * D + d0) = pack_bf16x2(o[0] * inv_l, o[1] * inv_l);
        }
    }
}

// Reductions across the four 16-lane rows of a wave (lanes j, j+16, j+32, j+48): v_permlane16_swap
// with the same register as both operands leaves lane (l & ~16)'s value in the first result and
// lane (l | 16)'s in the second, on every lane, so both lanes of a pair compute the same value.
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The key split with 16-row query blocks, for the smallest grids: twice as many workgroups as
// 32-row blocks give, so a single head of a few thousand tokens spreads over every compute
// unit.  The same walk as above (wave w takes tiles w, w+NW, ..., merge of the NW states at
// the end), on 16x16x32 bf16 MFMAs.  Lane l = 16 g + j works on query row j of the block:
//   S^T = K Q^T per 16-key block kb and 32-wide slice c of d: the K operand is key 16 kb + j,
//     dimensions 32 c + 8 g .. +8; Q's is row j, the same dimensions; accumulator register r
//     holds key 16 kb + 4 g + r of row j.
//   O^T += V^T P^T per 32-key chunk pc: the probabilities of blocks 2 pc and 2 pc + 1 that lane
//     l holds (keys 32 pc + 4 g + e and 32 pc + 16 + 4 g + e, e = 0..3) are its P^T operand,
//     and two LDS transpose reads give the V^T operand over the same keys for dimension
//     16 db + j; accumulator register r holds dimension 16 db + 4 g + r of row j.
template <int D, bool CAUSAL, bool PAD, bool OUT_F32, int NW>
__global__ void __launch_bounds__(64 * NW, 1) fa_fwd_bf16_ksplit16_kernel(FwdArgs a) {
    constexpr int BM = 16;                     // query rows per workgroup
    constexpr int BN = 64;                     // keys per tile
    constexpr int KC = D / 32;                 // k-steps of the S MFMA
    constexpr int NKB = BN / 16;               // 16-key blocks per tile
    constexpr int NDB = D / 16;                // 16-wide output blocks
    constexpr int PC = BN / 32;                // k-steps of the PV MFMA
    constexpr int RPW = 4 * NDB / NW;          // accumulator registers each wave finishes
    constexpr int KROWB = D * 2 + 16;          // K row stride in LDS (bytes): 16-byte pad
    constexpr int VSTR = D + 16;               // V row stride in LDS (bf16 elements): 32-byte pad
    constexpr int WBUFB = BN * KROWB + BN * VSTR * 2;   // bytes of one wave's K and V tiles
    constexpr int CPR = D * 2 / 16;            // 16-byte input chunks per row
    constexpr int LDC = BN * CPR / 64;         // chunks per lane per tensor per tile
    constexpr int MERGEB = (2 * NW * 16 + NW * NDB * 64 * 4) * 4;   // bytes of the merge state
    constexpr int SMEMB = NW * WBUFB > MERGEB ? NW * WBUFB : MERGEB;
    static_assert(LDC * 64 == BN * CPR, "a tile must split evenly over the 64 lanes");
    static_assert(RPW * NW == 4 * NDB && (RPW <= 4 ? 4 % RPW == 0 : RPW % 4 == 0), "whole register groups");
    static_assert(KROWB % 16 == 0 && WBUFB % 16 == 0, "16-byte LDS accesses stay aligned");
    static_assert(SMEMB <= 160 * 1024, "the tile buffers fit the LDS");

    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEMB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;
    const int g = lane >> 4;

    const TileCoord tc = tile_of(xcd_remap(blockIdx.x, a.total_wgs), a.n_qtiles, CAUSAL);
    const int b = tc.bh / a.H;
    const int N = a.N;
    const int q0 = tc.qt * BM;
    const int qrow = q0 + j;                   // the query row of this lane (every wave)
    const int64_t base = (int64_t)tc.bh * N * D;

    int Lk = N;
    if (PAD) {
        const int s = a.seqlens[b];
        Lk = s < 0 ? 0 : (s > N ? N : s);
    }
    if (Lk == 0) {  // every key masked: O = 0, LSE = -inf (written by wave 0; lane row j, d in [g D/4, (g+1) D/4))
        if (wave == 0 && qrow < N) {
            if (g == 0 && a.lse) a.lse[(int64_t)tc.bh * N + qrow] = kNegInf;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const int d0 = g * (D / 4) + 4 * c;
                if (OUT_F32) *(f32x4*)((float*)a.o + base + (int64_t)qrow * D + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
                else *(u32x2*)((uint16_t*)a.o + base + (int64_t)qrow * D + d0) = u32x2{0u, 0u};
            }
        }
        return;
    }

    int kv_end = Lk;
    if (CAUSAL) kv_end = kv_end < q0 + BM ? kv_end : q0 + BM;
    const int n_tiles = (kv_end + BN - 1) / BN;   // >= 1: key 0 is visible to every row

    // Q^T operand of k-step c: Q[qrow][32c + 8g .. +8]
    bf16x8 qf[KC];
    {
        const uint16_t* qp = (const uint16_t*)a.q + base + (int64_t)(qrow < N ? qrow : N - 1) * D + 8 * g;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            qf[c] = *(const bf16x8*)(qp + 32 * c);
            if (qrow >= N) qf[c] = bf16x8{};
        }
    }

    unsigned char* const ks = smem + wave * WBUFB;              // this wave's K tile (bytes)
    uint16_t* const vs = (uint16_t*)(ks + BN * KROWB);          // and V tile (bf16)
    const unsigned char* const kg = (const unsigned char*)a.k + base * 2;
    const unsigned char* const vg = (const unsigned char*)a.v + base * 2;
    // chunk ci = lane + 64 i of a tile: row ci / CPR, column chunk ci % CPR, loaded through
    // buffer resources that start at the tile and end at key N (rows past N read as zeros)
    int goff[LDC];
#pragma unroll
    for (int i = 0; i < LDC; ++i) {
        const int ci = lane + 64 * i;
        goff[i] = (ci / CPR) * D * 2 + (ci % CPR) * 16;
    }
    u32x4 kr[LDC], vr[LDC];   // the next tile on its way to LDS
    auto gload = [&](int tile) __attribute__((always_inline)) {
        const int64_t toff = static_cast<int64_t>(tile) * BN * D * 2;
        const int rec = (N - tile * BN) * D * 2;
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(kg + toff), (short)0, rec, 0x00020000);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(vg + toff), (short)0, rec, 0x00020000);
#pragma unroll
        for (int i = 0; i < LDC; ++i) {
            kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, goff[i], 0, 0));
            vr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, goff[i], 0, 0));
        }
    };
    auto swrite = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LDC; ++i) {
            const int ci = lane + 64 * i;
            const int row = ci / CPR;
            *(u32x4*)(ks + row * KROWB + (ci % CPR) * 16) = kr[i];
            *(u32x4*)(vs + row * VSTR + (ci % CPR) * 8) = vr[i];
        }
        // the wave's other lanes read what this lane wrote: wait for the writes to complete
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
    };
    // V^T operand of key chunk pc and output block db: the 16 lanes of row group g read the
    // 4-key x 16-dimension blocks at keys 32pc + 4g (and + 16), dimensions 16db; lane j gets
    // dimension 16db + j of those keys
    auto vt_frag = [&](int pc, int db) __attribute__((always_inline)) -> bf16x8 {
        const int row = 32 * pc + 4 * g + (j >> 2);
        const int col = 16 * db + 4 * (j & 3);
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + row * VSTR + col)));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + (row + 16) * VSTR + col)));
        return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };

    float m_run = kNegInf;   // running maximum of scale*log2(e)*s over this wave's visible keys
    float l_run = 0.f;       // this lane's running sum of 2^(.. - m_run) over its keys
    f32x4 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int n_rounds = (n_tiles + NW - 1) / NW;
    const int R = wave < n_tiles - (n_rounds - 1) * NW ? n_rounds : n_rounds - 1;
    auto tile_at = [&](int i) __attribute__((always_inline)) { return i * NW + wave; };
    auto tile_step = [&](int t, auto masked_c) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_c)::value;
        const int kv0 = t * BN;
        f32x4 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const bf16x8 kf = *(const bf16x8*)(ks + (16 * kb + j) * KROWB + 64 * c + 16 * g);
                s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], s[kb], 0, 0, 0);
            }
        }
        if constexpr (MASKED) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = kv0 + 16 * kb + 4 * g + r;
                    const bool ok = key < Lk && (!CAUSAL || key <= qrow);
                    s[kb][r] = ok ? s[kb][r] : kNegInf;
                }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = xor32_max(xor16_max(mx));
        // the scale is positive, so the largest score gives the largest scaled logit; a tile
        // without masked keys has a finite maximum
        const float m_tile = (MASKED && mx == kNegInf) ? kNegInf : mx * a.scale_log2;
        const float m_new = fmaxf(m_run, m_tile);
        const float m_use = (MASKED && m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float p = fast_exp2(fmaf(s[kb][r], a.scale_log2, -m_use));
                if constexpr (MASKED) p = s[kb][r] == kNegInf ? 0.f : p;   // exact zeros, also when scale == 0
                s[kb][r] = p;
                rs += p;
            }
        l_run = alpha * l_run + rs;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
        constexpr bool SPLIT = OUT_F32 || MASKED;
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) {
            const f32x4 p0 = s[2 * pc], p1 = s[2 * pc + 1];
            const u32x4 ph = {pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]),
                              pack_bf16x2(p1[0], p1[1]), pack_bf16x2(p1[2], p1[3])};
            u32x4 pl;
            if constexpr (SPLIT) {
                pl[0] = pack_bf16x2(p0[0] - bf16_lo_to_f32(ph[0]), p0[1] - bf16_hi_to_f32(ph[0]));
                pl[1] = pack_bf16x2(p0[2] - bf16_lo_to_f32(ph[1]), p0[3] - bf16_hi_to_f32(ph[1]));
                pl[2] = pack_bf16x2(p1[0] - bf16_lo_to_f32(ph[2]), p1[1] - bf16_hi_to_f32(ph[2]));
                pl[3] = pack_bf16x2(p1[2] - bf16_lo_to_f32(ph[3]), p1[3] - bf16_hi_to_f32(ph[3]));
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 vf = vt_frag(pc, db);
                acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8, ph), acc[db], 0, 0, 0);
                if constexpr (SPLIT)
                    acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8, pl), acc[db], 0, 0, 0);
            }
        }
    };
    // Step i computes tile i from LDS while the loads of tile i+1 are in flight, then moves
    // tile i+1 from registers to LDS
    if (R > 0) {
        gload(tile_at(0));
        swrite();
        for (int i = 0; i < R; ++i) {
            const bool more = i + 1 < R;
            if (more) gload(tile_at(i + 1));
            const int t = tile_at(i);
            if (t * BN + BN > Lk || (CAUSAL && t * BN + BN - 1 > q0)) tile_step(t, std::true_type{});
            else tile_step(t, std::false_type{});
            if (more) swrite();   // this tile's reads have all returned (their MFMAs used them)
        }
    }

    // merge.  LDS layout (floats): maxima [NW][16], sums [NW][16], accumulators
    // [NW][NDB][64][4] (block db of wave v at [v][db][lane], lane-contiguous 16-byte slots)
    __syncthreads();   // every wave is done with its tile buffers
    float* const ms = reinterpret_cast<float*>(smem);
    float* const ls = ms + NW * 16;
    float* const as = ls + NW * 16;
    const float l_tot = xor32_sum(xor16_sum(l_run));
    if (g == 0) {
        ms[wave * 16 + j] = m_run;
        ls[wave * 16 + j] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) *(f32x4*)(as + ((wave * NDB + db) * 64 + lane) * 4) = acc[db];
    __syncthreads();
    float m = kNegInf;
#pragma unroll
    for (int v = 0; v < NW; ++v) m = fmaxf(m, ms[v * 16 + j]);
    float sc[NW];
    float l = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const float mv = ms[v * 16 + j];
        sc[v] = mv == kNegInf ? 0.f : fast_exp2(mv - m);   // a wave without keys adds nothing
        l += sc[v] * ls[v * 16 + j];
    }
    if (qrow >= N) return;
    if (wave == 0 && g == 0 && a.lse) a.lse[(int64_t)tc.bh * N + qrow] = (m + __log2f(l)) * kLn2;
    const float inv_l = 1.0f / l;
    // wave w finishes accumulator registers x = RPW w .. RPW w + RPW - 1 (register x: block
    // x / 4, dimension 16 (x / 4) + 4 g + x % 4), in runs of up to four adjacent dimensions
    constexpr int RUN = RPW < 4 ? RPW : 4;
#pragma unroll
    for (int gi = 0; gi < RPW / RUN; ++gi) {
        const int x0 = RPW * wave + RUN * gi;
        const int db = x0 / 4, r0 = x0 % 4;
        float o[RUN];
#pragma unroll
        for (int u = 0; u < RUN; ++u) o[u] = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const float* src = as + ((v * NDB + db) * 64 + lane) * 4 + r0;
#pragma unroll
            for (int u = 0; u < RUN; ++u) o[u] += sc[v] * src[u];
        }
        const int d0 = 16 * db + 4 * g + r0;
        float* const of = (float*)a.o + base + (int64_t)qrow * D + d0;
        uint16_t* const ob = (uint16_t*)a.o + base + (int64_t)qrow * D + d0;
        if constexpr (RUN == 4) {
            if (OUT_F32) *(f32x4*)of = f32x4{o[0] * inv_l, o[1] * inv_l, o[2] * inv_l, o[3] * inv_l};
            else *(u32x2*)ob = u32x2{pack_bf16x2(o[0] * inv_l, o[1] * inv_l), pack_bf16x2(o[2] * inv_l, o[3] * inv_l)};
        } else {
            if (OUT_F32) *(f32x2*)of = f32x2{o[0] * inv_l, o[1] * inv_l};
            else *(uint32_t*)ob = pack_bf16x2(o[0] * inv_l, o[1] * inv_l);
        }
    }
}

}  // namespace fa
