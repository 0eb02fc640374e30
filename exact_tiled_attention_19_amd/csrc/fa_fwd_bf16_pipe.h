// Software-pipelined fused exact-attention forward for bf16 inputs on gfx950 (MI355X).
//
// Same mathematics as fa_fwd_bf16_kernel: for every query row the keys are consumed one tile
// at a time with a running maximum, a running sum of shifted exponentials and an unnormalised
// accumulator that are rescaled when the maximum moves ("FlashAttention Interview Questions:
// IO Complexity, Tiling, and Numerical Stability", section "How can softmax be computed across
// tiles?"), with S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 so every per-row
// statistic stays inside one lane (plus one exchange with lane^32).  What changes is how the
// work is arranged on the chip:
//
//   * One workgroup of four wave64s per (batch, head, 128-row query tile), 32 rows per wave,
//     two workgroups per CU (or eight waves and 256 rows, one workgroup per CU, for long
//     causal d = 128 heads).  Under the causal mask a workgroup runs the tile pair (t, n-1-t).
//   * Pipeline.  Iteration j has two phases.  Phase A issues the MFMAs of
//     S_{j+1}^T = K_{j+1} Q^T while the vector ALUs exponentiate the already shifted scores of
//     tile j, sum them and pack P_j to bf16.  Phase B issues O^T += V_j^T P_j^T while the vector
//     ALUs prepare tile j+1 (mask, row maximum, shift update, s*c - m).  P is produced and
//     consumed inside one iteration, so only the scores are double-buffered.  The iteration is
//     written as a fixed sequence of slots, one MFMA with its LDS read and a slice of vector
//     work each, kept in that order by sched_barrier.
//   * Shift policy.  With a bf16 output the shift follows the running row maximum, so the
//     key that dominates a row enters with probability exactly 1 and carries no bf16
//     rounding; a rise is left unapplied only while the new largest probability is at most a
//     quarter of the row's running sum and the rise is at most 8 (log2 units).  With a float32
//     output (P = P_hi + P_lo, two bf16 products) the shift is raised only when a row's tile
//     maximum exceeds it by more than 8, which skips most rescales.  Either way every
//     probability stays at most 2^8, and numerator and denominator share every shift, so the
//     result is unchanged.  The accumulator is rescaled (per row, applied wave-wide) whenever
//     some row's shift moves.
//   * Probability precision.  The value product takes P as one bf16 term (relative rounding
//     up to 2^-9) except where that error is not averaged away: a float32 output always uses
//     P_hi + P_lo, and with a bf16 output so do the masked tiles of a wave with a row that sees
//     fewer than one tile of keys (all of whose keys lie in masked tiles).  For such a row one
//     rounded probability could otherwise move the output by a few 1e-3 on top of the output's
//     own bf16 rounding; with a tile of keys or more the rounding errors average out.
//   * Direct-to-LDS loads.  K/V tiles move global -> LDS with buffer_load_dwordx4 ... lds.
//     Each instruction fills 1 KiB of LDS in lane order, so the bank-conflict-free layout is an
//     XOR swizzle of the 16-byte chunks of each row, realised by choosing which global chunk
//     each lane fetches.  Rows at or past N fall outside the buffer and read as zeros.
//   * Buffers.  K_{j+2} and V_{j+1} are loaded during iteration j into the buffers whose
//     contents (K_j, V_{j-1}) were last read in iteration j-1; one barrier per iteration.
#pragma once

#include <type_traits>

#include "fa_fwd_bf16.h"
#include "fa_dropout.h"

namespace fa {

// XOR swizzles of the 16-byte chunk index within a K or V row (row = key index in the tile).
// K is read as 32 rows x one chunk per MFMA operand, V as 4 rows x 64 bytes per transpose
// read; these spread both patterns over all LDS banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
    return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// Swizzle of the 16-byte chunks of an 8-bit K row (D bytes): a lane reads 32 bytes (two
// chunks) of row l32 per k-step.  LDS serves 16-byte reads 16 lanes (256 bytes, all 64 banks)
// at a time; the 16 rows such a group reads then fall on 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int swz_k8(int row) {
    return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ u32x8 u32x8_of(u32x4 lo, u32x4 hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

// One S-product step: 32 keys x 32 query rows over 16 (bf16) or 64 (FP8 E4M3) head dimensions.
// The 8-bit form is v_mfma_f32_32x32x64_f8f6f4 (operand formats 0 = E4M3, block scales off).
__device__ __forceinline__ f32x16 mfma_s(bf16x8 kf, bf16x8 qf, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_s(i32x8 kf, i32x8 qf, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf, c, 0, 0, 0, 0, 0, 0);
}

// Four E4M3 codes (one dword) -> four bf16 (two dwords); every E4M3 value is a bf16 value.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w) {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

// IEEE maximum without the canonicalising moves fmaxf needs (v_maximum3_f32 on gfx950).  The
// scores reduced with it are finite or -inf, so NaN handling does not arise.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max(a, b, c) as one v_maximum3_f32 (register operands only).  Written out because, given the
// running-maximum chain m = max(m, max(a, b)), the compiler rebuilds it as a tree whose leaves
// are two-input maxima: 24 instructions per 32 scores instead of 16.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_maximum3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// 16 bytes per lane from a buffer resource straight into LDS (buffer_load_dwordx4 ... lds):
// lane i's data lands at lds + 16 i.  A device function, not a lambda, because the builtin
// exists only for the device.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// The four K/V tile buffers in LDS: one object per (size, id), shared by every instantiation of
// pipe_tile with that tile size, so a kernel that runs two instantiations does not double its
// LDS.  Distinct objects (not offsets into one array) let the compiler see that an outstanding
// global->LDS load into one buffer does not alias LDS reads from another.
template <int TILEB, int ID>
__device__ __forceinline__ unsigned char* pipe_lds() {
    __shared__ __attribute__((aligned(1024))) unsigned char buf[TILEB];
    return buf;
}

// One query tile (BM rows of head bh) from start to finish; the kernels below run one or two.
// VL: the rows belong to one sequence of a packed batch described by `sg` (token-major rows,
// own query and key lengths, causal diagonal offset); otherwise the [B, H, N, d] layout.
// SPLITM: the masked steps take two-term probabilities (a tile with a row that sees fewer than
// BN keys).  NW: waves per workgroup (4, or 8 for one 256-row workgroup per CU).  DROP:
// dropout on the probabilities that enter the value product (the row sums, and so O's
// normaliser and the log-sum-exp, take them undropped; kept ones are scaled in the epilogue).
// STF32: the output rows are stored as float32 whatever OUT_F32 says about the probabilities'
// precision (the key ranges of the split packed kernel, merged and rounded afterwards).
template <int D, int BN, int RB, bool CAUSAL, bool PAD, bool OUT_F32, bool VL = false, bool SPLITM = false, int NW = 4,
          bool DROP = false, bool F8 = false, bool STF32 = OUT_F32>
__device__ __forceinline__ void pipe_tile(const FwdArgs& a, int bh, int qt, const SeqGeom& sg = SeqGeom{}) {
    constexpr int WR = 32 * RB;             // query rows per wave
    constexpr int BM = NW * WR;             // query rows per workgroup
    constexpr int KC = F8 ? D / 64 : D / 16;  // k-steps of the S MFMA
    constexpr int NKB = BN / 32;            // 32-key blocks per tile
    constexpr int NDB = D / 32;             // 32-wide output blocks
    constexpr int PC = BN / 16;             // k-steps of the PV MFMA
    constexpr int ESZ = F8 ? 1 : 2;         // bytes per input element
    constexpr int KROWB = D * ESZ;          // bytes per K row in LDS (no padding)
    constexpr int ROWB = D * 2;             // bytes per V row in LDS (bf16; 8-bit V is widened)
    constexpr int KTILEB = BN * KROWB;      // bytes per K tile
    constexpr int TILEB = BN * ROWB;        // bytes per V tile
    constexpr int CPR = KROWB / 16;         // 16-byte chunks per input row
    constexpr int LPW = KTILEB / 1024 / NW; // 1 KiB loads per wave per K (and per V) tile
    using KFrag = std::conditional_t<F8, i32x8, bf16x8>;   // S operand fragment
    constexpr bool PRECISE = OUT_F32;
    // Shift threshold (log2 units).  With a bf16 output the probabilities enter the PV product
    // as single bf16 values, so the shift tracks the exact row maximum (threshold 0: the largest
    // probability is then exactly 1 and carries no rounding); with the two-term split used for
    // a float32 output a shift lagging by up to 8 costs nothing.
    constexpr float kTau = PRECISE ? 8.0f : 0.0f;
    // Largest rise of the row maximum (log2 units) that the bf16-output rule below may leave
    // unapplied; the float32-output threshold kTau bounds the probabilities by the same 2^8.
    constexpr float kSkipCap = 8.0f;
    static_assert(LPW >= 1 && LPW * NW * 1024 == KTILEB, "tile must split into 1 KiB pieces");
    static_assert(!F8 || (!DROP && !VL && RB == 1), "8-bit inputs: fixed-length heads without dropout");
    static_assert(!DROP || (RB == 1 && BN == 64 && !VL), "dropout words are laid out for one 32-row block");

    unsigned char* const kbuf0 = pipe_lds<KTILEB, 0>();
    unsigned char* const kbuf1 = pipe_lds<KTILEB, 1>();
    unsigned char* const vbuf0 = pipe_lds<TILEB, 2>();
    unsigned char* const vbuf1 = pipe_lds<TILEB, 3>();
    constexpr int KB0 = 0, KB1 = 1, VB0 = 2, VB1 = 3;
    auto buf = [&](int id) __attribute__((always_inline)) -> unsigned char* {
        return id == KB0 ? kbuf0 : id == KB1 ? kbuf1 : id == VB0 ? vbuf0 : vbuf1;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const TileCoord tc{bh, qt};
    const int b = tc.bh / a.H;
    const int N = VL ? sg.Lq : a.N;            // query rows of this head
    const int q0 = tc.qt * BM;
    const int qw0 = q0 + wave * WR;          // first query row of this wave
    int qrow[RB];                            // the rows this lane's statistics belong to
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) qrow[rb] = qw0 + 32 * rb + l32;
    const int64_t base = VL ? sg.qbase : (int64_t)tc.bh * N * D;   // query / output rows
    const int64_t kbase = VL ? sg.kbase : base;                       // key / value rows
    const int64_t lbase = VL ? sg.lbase : (int64_t)tc.bh * N;         // log-sum-exp entries
    const int64_t obase = VL ? sg.obase : base;                       // output rows
    const int RSE = VL ? sg.rse : D;           // elements between consecutive rows
    const int ORSE = VL ? sg.orse : D;         // the same for the output
    const int RSB = RSE * ESZ;                 // the same in bytes (inputs)
    const int dlt = VL ? sg.dlt : 0;           // causal: key j visible to row i iff j <= i + dlt

    int Lk = N;
    if (VL) {
        Lk = sg.Lk;
    } else if (PAD) {
        const int s = a.seqlens[b];
        Lk = s < 0 ? 0 : (s > N ? N : s);
    }
    if (Lk == 0) {  // every key masked: O = 0, LSE = -inf
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (qrow[rb] >= N) continue;
            if (hh == 0 && a.lse) a.lse[lbase + qrow[rb]] = kNegInf;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = 32 * db + 8 * j + 4 * hh;
                    if (STF32) *(f32x4*)((float*)a.o + obase + (int64_t)qrow[rb] * ORSE + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
                    else *(u32x2*)((uint16_t*)a.o + obase + (int64_t)qrow[rb] * ORSE + d0) = u32x2{0u, 0u};
                }
        }
        return;
    }

    // The causal limits below use the diagonal offset dlt, which is 0 for the [B, H, N, d]
    // layout; there the original expressions are kept (every term is non-negative).
    int kv_end = Lk;
    if (CAUSAL) {
        if constexpr (VL) {
            kv_end = kv_end < q0 + BM + dlt ? kv_end : q0 + BM + dlt;
            kv_end = kv_end > 0 ? kv_end : 0;
        } else {
            kv_end = kv_end < q0 + BM ? kv_end : q0 + BM;
        }
    }
    const int n_tiles = (kv_end + BN - 1) / BN;
    // tiles this wave computes: under the causal mask the last tiles may lie entirely above
    // this wave's rows and carry no visible key for any of them
    int n_w = n_tiles;
    if (CAUSAL) {
        int lim;
        if constexpr (VL) {
            const int x = qw0 + WR - 1 + dlt;   // last key visible to the wave's last row
            lim = x < 0 ? 0 : x / BN + 1;
        } else {
            lim = (qw0 + WR - 1) / BN + 1;
        }
        n_w = lim < n_w ? lim : n_w;
    }
    if (VL && qw0 >= N) n_w = 0;               // a wave past the sequence's last query row
    // tiles [0, n_plain) need no mask for any row of this wave
    int n_plain = Lk / BN;
    if (CAUSAL) {
        int c;                                  // tiles whose last key the wave's first row sees
        if constexpr (VL) {
            const int x = qw0 + 1 + dlt;
            c = x < 0 ? 0 : x / BN;
        } else {
            c = (qw0 + 1) / BN;
        }
        n_plain = c < n_plain ? c : n_plain;
    }

    // Q^T operand fragments (B operand of the S MFMA), kept in VGPRs for the whole kernel
    KFrag qf[RB][KC];
    if constexpr (F8) {
        // the same byte -> dimension assignment as the K fragments below: lane half hh takes
        // bytes 64c + 32hh .. 64c + 32hh + 31 of its row in k-step c; the MFMA sums over all
        // 64 positions of a step whatever its internal order, so Q and K need only agree
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const unsigned char* qp = (const unsigned char*)a.q + base + (int64_t)(qrow[rb] < N ? qrow[rb] : N - 1) * RSE + 32 * hh;
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const u32x4 lo = *(const u32x4*)(qp + 64 * c);
                const u32x4 hi = *(const u32x4*)(qp + 64 * c + 16);
                qf[rb][c] = __builtin_bit_cast(i32x8, u32x8_of(lo, hi));
                if (qrow[rb] >= N) qf[rb][c] = KFrag{};
            }
        }
    } else
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const uint16_t* qp = (const uint16_t*)a.q + base + (int64_t)(qrow[rb] < N ? qrow[rb] : N - 1) * RSE + 8 * hh;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            qf[rb][c] = *(const bf16x8*)(qp + 16 * c);
            if (qrow[rb] >= N) qf[rb][c] = bf16x8{};
        }
    }

    // ---- direct-to-LDS tile loads ---------------------------------------------------------
    // Piece r (1 KiB) of a tile holds rows 4r .. 4r+3 (D = 128) or 8r .. 8r+7 (D = 64).  Lane
    // lam writes physical chunk p = 64 r + lam, i.e. row p / CPR, chunk p % CPR, and fetches the
    // logical chunk that the swizzle maps there.  The buffer's byte range ends with the last
    // key row, so rows past it read as zeros (for the packed layout: the last row's end).
    const int64_t krec = VL ? (int64_t)(Lk - 1) * RSB + KROWB : (int64_t)N * KROWB;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const unsigned char*)a.k + kbase * ESZ), (short)0, (int)(uint32_t)krec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const unsigned char*)a.v + kbase * ESZ), (short)0, (int)(uint32_t)krec, 0x00020000);
    // 8-bit V takes a register round trip instead: lane lam loads the 16 codes of chunk p of
    // the tile (row p / CPR, dimensions 16 (p % CPR) ..), widens them to bf16 and writes the
    // two bf16 chunks 2 (p % CPR) and 2 (p % CPR) + 1 of that row into the bf16 V layout
    uint32_t koff[LPW], voff[LPW], vws[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int p = (i * NW + wave) * 64 + lane;
        const int row = p / CPR;
        const int pch = p % CPR;
        koff[i] = row * RSB + (pch ^ (F8 ? swz_k8<D>(row) : swz_k<D>(row))) * 16;
        voff[i] = row * RSB + (F8 ? pch : (pch ^ swz_v<D>(row))) * 16;
        vws[i] = row * ROWB + ((2 * pch) ^ swz_v<D>(row)) * 16;   // chunk 2 pch + 1 follows it
    }
    // Rows whose starts share LDS banks (256 / ROWB rows apart: the next row at d = 128, the one
    // after at d = 64) write their two chunks in opposite orders, so that each write of a group
    // of 16 lanes covers 16 distinct 16-byte bank groups.  Every piece starts on a row that is a
    // multiple of 8, so the lane alone decides.
    const bool v8_swap = (((lane / CPR) >> (ROWB == 256 ? 0 : 1)) & 1) != 0;
    auto store_v8 = [&](const u32x4 (&raw)[LPW], int vbuf_id) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const u32x2 w0 = e4m3x4_to_bf16(raw[i][0]), w1 = e4m3x4_to_bf16(raw[i][1]);
            const u32x2 w2 = e4m3x4_to_bf16(raw[i][2]), w3 = e4m3x4_to_bf16(raw[i][3]);
            const u32x4 lo = u32x4{w0[0], w0[1], w1[0], w1[1]}, hi = u32x4{w2[0], w2[1], w3[0], w3[1]};
            *(u32x4*)(buf(vbuf_id) + vws[i] + (v8_swap ? 16 : 0)) = v8_swap ? hi : lo;
            *(u32x4*)(buf(vbuf_id) + vws[i] + (v8_swap ? 0 : 16)) = v8_swap ? lo : hi;
        }
    };
    auto load_tile = [&](auto is_v, int tile, int buf_off) __attribute__((always_inline)) {
        constexpr bool IS_V = decltype(is_v)::value;
        const uint32_t t0 = (uint32_t)tile * (uint32_t)(BN * RSB);
        if constexpr (F8 && IS_V) {
            u32x4 raw[LPW];
#pragma unroll
            for (int i = 0; i < LPW; ++i)
                raw[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[i] + t0, 0, 0));
            store_v8(raw, buf_off);
        } else {
#pragma unroll
            for (int i = 0; i < LPW; ++i)
                buffer_load_lds16(IS_V ? vrs : krs, buf(buf_off) + (i * NW + wave) * 1024,
                                  (IS_V ? voff[i] : koff[i]) + t0);
        }
    };

    // ---- LDS read addresses (bytes within a tile buffer) -----------------------------------
    // K operand of k-step c, block kb: row 32kb + l32, logical chunk 2c + hh.
    // 8-bit K: k-step c, lane half hh reads logical chunks 4c + 2hh and 4c + 2hh + 1 (kaddr,
    // kaddr2), the bytes the Q fragment holds.
    const int krow_base = l32 * KROWB;
    const int kswz = (F8 ? swz_k8<D>(l32) : swz_k<D>(l32)) * 16;   // 32kb + l32 has the same swizzle as l32
    int kaddr[KC], kaddr2[KC];                // byte offset of k-step c's chunk(s) in row l32
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        if constexpr (F8) {
            kaddr[c] = krow_base + (((4 * c + 2 * hh) * 16) ^ kswz);
            kaddr2[c] = krow_base + (((4 * c + 2 * hh + 1) * 16) ^ kswz);
        } else {
            kaddr[c] = krow_base + (((2 * c + hh) * 16) ^ kswz);
            kaddr2[c] = kaddr[c];
        }
    }
    // V^T operand (transpose read) of chunk pc, block db: row 16pc + 4hh + (l32 & 15) / 4 (+8),
    // logical column 32db + (l32 & 16) + 4 (l32 & 3) -> chunk 4db + ((l32 & 16) >> 3) +
    // ((l32 & 3) >> 1), byte (l32 & 1) * 8 within the chunk.
    const int vrow = 4 * hh + ((l32 & 15) >> 2);
    const int vswz = swz_v<D>(vrow);
    const int vcl = ((l32 & 16) >> 3) + ((l32 & 3) >> 1);
    int vaddr[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) vaddr[db] = vrow * ROWB + (((4 * db + vcl) ^ vswz) * 16) + (l32 & 1) * 8;

    auto tile_rsrc = [&](const void* t, int64_t off, int tile) __attribute__((always_inline)) {
        const int64_t start = (int64_t)tile * BN * RSB;         // bytes into this head
        const int64_t left = krec - start;
        return __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)t + off * ESZ + start),
                                                 (short)0, left > 0 ? (int)(uint32_t)left : 0, 0x00020000);
    };

    auto kfrag_at = [&](int kbuf, int c, int kb) __attribute__((always_inline)) -> KFrag {
        const unsigned char* p = buf(kbuf) + kb * 32 * KROWB;
        if constexpr (F8)
            return __builtin_bit_cast(i32x8, u32x8_of(*(const u32x4*)(p + kaddr[c]), *(const u32x4*)(p + kaddr2[c])));
        else
            return *(const bf16x8*)(p + kaddr[c]);
    };
    auto compute_s = [&](f32x16 (&s)[RB][NKB], int kbuf) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[rb][kb] = f32x16{};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const KFrag kf = kfrag_at(kbuf, c, kb);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) s[rb][kb] = mfma_s(kf, qf[rb][c], s[rb][kb]);
            }
        }
    };

    float m_run[RB], l_run[RB], alpha_pend[RB];
    f32x16 acc[RB][NDB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = kNegInf;     // exponent shift (log2 units), raised lazily
        l_run[rb] = 0.f;         // this lane half's running sum of 2^(scaled score - m_run)
        alpha_pend[rb] = 1.f;    // factor the accumulator owes before the next PV product
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[rb][db] = f32x16{};
    }
    bool rescale_pend = false;
    // Heavy-tile test (bf16 output, one-term probabilities), for the tile whose scores were last
    // prepared: 1 when that tile's row maximum became the shift and lies in this lane half (its
    // key's probability is then 1 up to a float32 rounding, exact in bf16), else 0.
    float one_pend[RB];
    // Whether this lane half of the current tile is heavy (its P_lo is used; other lanes add
    // exactly zero).
    bool hv_lane[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        one_pend[rb] = 0.f;
        hv_lane[rb] = false;
    }

    // Multiplier of the masked steps' fma: scale*log2(e), or the smallest normal float when the
    // scale is 0 (then every visible t is within 1e-30 of 0, as it should be, and -inf * c
    // stays -inf instead of NaN).
    const float c_mask = a.scale_log2 > 0.f ? a.scale_log2 : 1.17549435e-38f;

    // Phase B vector work for tile `tile`: mask (edge tiles only), row maximum, lazy shift
    // update, then the shifted scores t = s * scale * log2(e) - m in place.
    auto prep = [&](f32x16 (&s)[RB][NKB], int tile, bool masked) __attribute__((always_inline)) {
        const int kv0 = tile * BN;
        if (masked) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                        const bool ok = key < Lk && (!CAUSAL || key <= qrow[rb] + dlt);
                        s[rb][kb][r] = ok ? s[rb][kb][r] : kNegInf;
                    }
        }
        float m_tile[RB];
        bool need[RB];
        bool need_any = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float mx = s[rb][0][0];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = vmax(mx, s[rb][kb][r]);
            const float hmx = mx;
            mx = xor32_max(mx);
            m_tile[rb] = (mx == kNegInf) ? kNegInf : mx * a.scale_log2;
            need[rb] = m_tile[rb] > m_run[rb] + kTau;     // per row: the update depends on
            need_any = need_any || need[rb];              // this row's scores only
            one_pend[rb] = (need[rb] && hmx == mx) ? 1.f : 0.f;
        }
        const bool any = __builtin_amdgcn_ballot_w64(need_any) != 0;   // wave-uniform
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float m_new = need[rb] ? m_tile[rb] : m_run[rb];
            const float alpha = (m_new == m_run[rb]) ? 1.f : fast_exp2(m_run[rb] - m_new);
            m_run[rb] = m_new;
            l_run[rb] *= alpha;          // l holds tiles < tile, all in the old shift
            alpha_pend[rb] = alpha;      // acc still receives P V of the previous tile first
            const float nm = (m_new == kNegInf) ? 0.f : -m_new;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float t = fmaf(s[rb][kb][r], a.scale_log2, nm);
                    // hidden keys stay -inf (their weight is exactly 0), also when scale == 0
                    s[rb][kb][r] = (masked && s[rb][kb][r] == kNegInf) ? kNegInf : t;
                }
        }
        rescale_pend = any;
    };

    auto rescale_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[rb][db] *= alpha_pend[rb];
    };

    constexpr int NSF = KC * NKB;                       // K fragments per tile
    constexpr int NPF = PC * NDB;                       // V fragments per tile
    // Scheduling pattern of the prologue's S product: each fragment's LDS read is issued one
    // fragment ahead of its MFMA, so its latency is covered by the previous MFMA and the reads
    // are not all hoisted to the top (which would keep every operand live at once); VS vector
    // instructions ride along with each MFMA.
    auto pattern_s = [](auto vs_c) __attribute__((always_inline)) {
        constexpr int VS = decltype(vs_c)::value;
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int i = 0; i < NSF - 1; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
            for (int m = 0; m < RB; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if constexpr (VS > 0) __builtin_amdgcn_sched_group_barrier(0x002, VS, 0);
            }
        }
#pragma unroll
        for (int m = 0; m < RB; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if constexpr (VS > 0) __builtin_amdgcn_sched_group_barrier(0x002, VS, 0);
        }
    };
    using V0 = std::integral_constant<int, 0>;

    f32x16 sA[RB][NKB], sB[RB][NKB];
    u32x4 ph[RB][PC], pl[RB][PC];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) pl[rb][pc] = u32x4{};

    auto wait_loads = []() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)

    // ---- steady-state iteration, written in issue order -----------------------------------
    // The iteration is a fixed sequence of slots.  A phase-A slot reads the next K fragment
    // from LDS, issues the S MFMA(s) of the current one and a fixed slice of tile j's
    // exponentials / sums / packing; a phase-B slot does the same with V fragments, the PV
    // MFMA(s) and a slice of tile j+1's preparation.  sched_barrier(0) between slots keeps the
    // compiler from regrouping them, so every MFMA has vector work beside it and every LDS
    // read has one MFMA of time before its data is needed.
    constexpr int NE = 16 * NKB;            // scores per lane per tile (and row block)
    constexpr int EA = NE / NSF;            // elements exponentiated per phase-A slot
    constexpr int HB = NPF / 2;             // phase-B slots spent on the row maximum
    constexpr int EM = NE / HB;             // elements folded into the maximum per slot
    constexpr int NFMA = NPF - HB - 1;      // phase-B slots left for s*c - m
    static_assert(EA * NSF == NE && EM * HB == NE && EA % 2 == 0, "slot split");
    static_assert(2 * LPW <= NSF, "every K and V load of a tile needs a phase-A slot");
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    auto kfrag = [&](int kbuf, int i) __attribute__((always_inline)) -> KFrag {
        return kfrag_at(kbuf, i / NKB, i % NKB);
    };
    auto vfrag = [&](int vbuf, int i) __attribute__((always_inline)) -> bf16x8 {
        const int pc = i / NDB, db = i % NDB;
        const unsigned char* p0 = buf(vbuf) + vaddr[db] + pc * 16 * ROWB;
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 8 * ROWB)));
        return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    // The heavy tile's second term (see fast_body): P_lo = p - bf16(p), from the probabilities
    // that phase A left in the score registers of parity PAR, times that tile's V (buffer PAR,
    // refilled only after the iteration's closing barrier), for the lane halves found heavy; the
    // others contribute exactly 0.
    auto heavy_fix = [&](auto par_c) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_c)::value;
        f32x16 (&sp)[RB][NKB] = PAR == 0 ? sA : sB;
        constexpr int VB_T = PAR == 0 ? VB0 : VB1;
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) {
            u32x4 lo[RB];   // this k-step's P_lo only (the register budget decides occupancy)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int f = 8 * pc + 2 * w, fk = f / 16, fr = f % 16;
                    const float h0 = bf16_lo_to_f32(ph[rb][pc][w]), h1 = bf16_hi_to_f32(ph[rb][pc][w]);
                    float r0 = sp[rb][fk][fr] - h0, r1 = sp[rb][fk][fr + 1] - h1;
                    if constexpr (DROP) {   // a dropped key entered as 0: its residual is 0 too
                        r0 = h0 == 0.f ? 0.f : r0;
                        r1 = h1 == 0.f ? 0.f : r1;
                    }
                    r0 = hv_lane[rb] ? r0 : 0.f;
                    r1 = hv_lane[rb] ? r1 : 0.f;
                    lo[rb][w] = pack_bf16x2(r0, r1);
                }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 v2 = vfrag(VB_T, pc * NDB + db);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v2, __builtin_bit_cast(bf16x8, lo[rb]),
                                                                          acc[rb][db], 0, 0, 0);
            }
        }
    };

    auto fast_body = [&](auto par_c, auto masked_c, auto split_c, int j) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_c)::value;
        constexpr bool MASKED = decltype(masked_c)::value;
        // two-term probabilities for tile j: always with a float32 output; with a bf16 output
        // when the caller asks (masked tiles of a wave whose rows see fewer than BN keys)
        constexpr bool SPLIT = PRECISE || decltype(split_c)::value;
        f32x16 (&s_cur)[RB][NKB] = PAR == 0 ? sA : sB;
        f32x16 (&s_nxt)[RB][NKB] = PAR == 0 ? sB : sA;
        constexpr int KB_THIS = PAR == 0 ? KB0 : KB1, KB_OTHER = PAR == 0 ? KB1 : KB0;
        constexpr int VB_THIS = PAR == 0 ? VB0 : VB1, VB_OTHER = PAR == 0 ? VB1 : VB0;
        // buffer resources starting at tiles j+2 (K) and j+1 (V): the tile offset goes into the
        // scalar base address, so the per-lane offsets need no vector add; the record count
        // shrinks accordingly and keeps rows past N reading as zeros
        const __amdgpu_buffer_rsrc_t krs_t = tile_rsrc(a.k, kbase, j + 2);
        const __amdgpu_buffer_rsrc_t vrs_t = tile_rsrc(a.v, kbase, j + 1);
        int vis[RB];   // masked tiles: keys of tile j+1 at offset < vis are visible to the row
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            int lim = Lk;
            if (CAUSAL) lim = lim < qrow[rb] + 1 + dlt ? lim : qrow[rb] + 1 + dlt;
            vis[rb] = lim - (j + 1) * BN - 4 * hh;
        }
        float rs[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) rs[rb][0] = rs[rb][1] = 0.f;
        // dropout words of the current 32-key half of tile j (see dropout_words_fwd)
        uint32_t dw[4];
        // phase A
        KFrag kf = kfrag(KB_OTHER, 0);
        KFrag kf1 = kfrag(KB_OTHER, 1);
        u32x4 vraw[LPW];   // 8-bit V tile j+1, widened and stored after phase B
#pragma unroll
        for (int i = 0; i < NSF; ++i) {
            if (i < LPW) buffer_load_lds16(krs_t, buf(KB_THIS) + (i * NW + wave) * 1024, koff[i]);
            else if (i < 2 * LPW) {
                if constexpr (F8)
                    vraw[i - LPW] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs_t, voff[i - LPW], 0, 0));
                else
                    buffer_load_lds16(vrs_t, buf(VB_OTHER) + ((i - LPW) * NW + wave) * 1024, voff[i - LPW]);
            }
            KFrag kf2 = kf1;            // operands are read two fragments ahead
            if (i + 2 < NSF) kf2 = kfrag(KB_OTHER, i + 2);
            const int c = i / NKB, kb = i % NKB;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                s_nxt[rb][kb] = mfma_s(kf, qf[rb][c], c == 0 ? f32x16{} : s_nxt[rb][kb]);
            if constexpr (DROP) {
                if ((i * EA) % 16 == 0)   // first slot of a 32-key half
                    dropout_words_fwd(dw, j * BN, (i * EA) / 16, qrow[0], hh, tc.bh, a.drop_offset, a.drop_k0, a.drop_k1);
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int e = 0; e < EA; e += 2) {
                    const int f = i * EA + e, fk = f / 16, fr = f % 16;
                    const float p0 = fast_exp2(s_cur[rb][fk][fr]);
                    const float p1 = fast_exp2(s_cur[rb][fk][fr + 1]);
                    s_cur[rb][fk][fr] = p0;
                    s_cur[rb][fk][fr + 1] = p1;
                    rs[rb][(e / 2) & 1] += p0 + p1;
                    float d0 = p0, d1 = p1;      // the probabilities entering the value product
                    if constexpr (DROP) {
                        d0 = drop_keep(dw[fr / 4], fr % 4, a.drop_t) ? p0 : 0.f;
                        d1 = drop_keep(dw[fr / 4], fr % 4 + 1, a.drop_t) ? p1 : 0.f;
                    }
                    const int pc = f / 8, w = (f % 8) / 2;
                    ph[rb][pc][w] = pack_bf16x2(d0, d1);
                    if constexpr (SPLIT)
                        pl[rb][pc][w] = pack_bf16x2(d0 - bf16_lo_to_f32(ph[rb][pc][w]), d1 - bf16_hi_to_f32(ph[rb][pc][w]));
                }
            kf = kf1;
            kf1 = kf2;
            __builtin_amdgcn_sched_barrier(0);
        }
        // Heavy tile (bf16 output, one-term probabilities).  A probability rounded to bf16 errs by
        // up to 2^-8 of itself, which stays far inside the output's bound for keys of small
        // weight, but a key that ends with a large share of its row (two near-equal dominant
        // keys, say) can move O by a few 1e-3: too much where |O| is in [2, 4) and the output's
        // own rounding already takes up to 7.8e-3 of the 1e-2 bound.  So a lane half whose keys
        // of tile j may end with more than a quarter of the row's weight -- a probability above
        // l/4, with l the row sum including tile j, which can only grow -- also gets P_lo =
        // p - bf16(p), in an extra value product after phase B (run when any lane needs it; the
        // other lanes add exactly 0, so every row's result depends on its own scores only).
        // The bound on one key's probability is the half's share of the tile's sum, less the
        // exact 1 of the shift's own maximum when it lies in this half, and at most 1 (the shift
        // is at or above every score of the tile, or else, by the rescale rule, every
        // probability of the tile is at most l/4 already).  The test and the extra product
        // (heavy_fix) run between the phases, while the probabilities are still in registers.
        constexpr bool DYN = !SPLIT;
        float rsum[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            rsum[rb] = rs[rb][0] + rs[rb][1];
            l_run[rb] += rsum[rb];
        }
        float l_all[RB];   // the whole row's running sum (both lane halves), tiles <= j
        if constexpr (DYN) {
            const float wmul_h = DROP ? 4.f * a.drop_keep_scale : 4.f;   // kept keys weigh 1/(1-p) more
            bool small_any = false;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                l_all[rb] = xor32_sum(l_run[rb]);
                small_any = small_any || l_all[rb] < wmul_h;   // the test can only pass when l < 4
            }
            // Phase A's results feed phase B; without these (empty) uses the compiler would sink
            // their computation past the branches below, away from the MFMAs of phase A.
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int pc = 0; pc < PC; ++pc) asm volatile("" : "+v"(ph[rb][pc]));
                asm volatile("" : "+v"(l_run[rb]), "+v"(l_all[rb]));
            }
            bool heavy = false;
            if (__builtin_amdgcn_ballot_w64(small_any) != 0) {
                bool hv_any = false;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    hv_lane[rb] = fminf(rsum[rb] - one_pend[rb], 1.f) * wmul_h > l_all[rb];
                    hv_any = hv_any || hv_lane[rb];
                }
                heavy = __builtin_amdgcn_ballot_w64(hv_any) != 0;
            }
            if (heavy) heavy_fix(par_c);
        }
        // phase B
        float mx[RB][2];
        bf16x8 vf = vfrag(VB_THIS, 0);
        bf16x8 vf1 = vfrag(VB_THIS, 1);
#pragma unroll
        for (int i = 0; i < NPF; ++i) {
            bf16x8 vf2 = vf1;
            if (i + 2 < NPF) vf2 = vfrag(VB_THIS, i + 2);
            const int pc = i / NDB, db = i % NDB;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, ph[rb][pc]), acc[rb][db], 0, 0, 0);
                if constexpr (SPLIT)
                    acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, pl[rb][pc]), acc[rb][db], 0, 0, 0);
            }
            if (i < HB) {
                // fold EM scores of tile j+1 into two running maxima (masked tiles: hidden keys
                // first become -inf; key 32kb + 8(r/4) + 4hh + r%4 of the tile is visible to
                // this lane's row iff its offset is below vis[rb] - 4hh)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < EM; e += 2) {
                        const int f = i * EM + e, fk = f / 16, fr = f % 16;
                        const int h = (e / 2) & 1;
                        if constexpr (MASKED) {
#pragma unroll
                            for (int u = 0; u < 2; ++u) {
                                const int off = 32 * fk + 8 * ((fr + u) >> 2) + ((fr + u) & 3);
                                s_nxt[rb][fk][fr + u] = off < vis[rb] ? s_nxt[rb][fk][fr + u] : kNegInf;
                            }
                        }
                        const float a0 = s_nxt[rb][fk][fr], a1 = s_nxt[rb][fk][fr + 1];
                        mx[rb][h] = (i == 0 && e < 4) ? vmax(a0, a1) : vmax3(mx[rb][h], a0, a1);
                    }
            } else if (i == HB) {
                bool need[RB];
                bool need_any = false;
                float m_tile[RB];
                if constexpr (!PRECISE && !DYN) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) l_all[rb] = xor32_sum(l_run[rb]);
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const float hmx = vmax(mx[rb][0], mx[rb][1]);
                    const float m = xor32_max(hmx);
                    m_tile[rb] = m * a.scale_log2;
                    if constexpr (PRECISE) {
                        need[rb] = m_tile[rb] > m_run[rb] + kTau;
                    } else {
                        // bf16 probabilities: a raised maximum moves the shift (so that the new
                        // largest probability is exactly 1) unless that probability, 2^(m_tile -
                        // m_run), is at most a quarter of the row's running sum.  Such a key keeps
                        // a weight of at most 1/4 in the output, and its bf16 rounding then counts
                        // like that of any other key; the rescale is skipped.  Every key that
                        // dominates a row still enters with probability exactly 1.  The sum is
                        // the whole row's (both lane halves), so both halves decide alike.
                        // With dropout a kept key's weight is further multiplied by the keep scale.
                        // The skip is capped: a rise of more than kSkipCap always moves the
                        // shift, so every probability stays at most 2^kSkipCap and the sum at
                        // most that times the key count.  Without the cap, logits that climb a
                        // little per tile (each rise small against the grown sum) never move
                        // the shift, and the sum overflows float32 once the climb passes
                        // about 88 nats (2^128).
                        const float wmul = DROP ? 4.f * a.drop_keep_scale : 4.f;
                        const float rise = m_tile[rb] - m_run[rb];
                        need[rb] = rise > 0.f && (rise > kSkipCap || fast_exp2(rise) * wmul > l_all[rb]);
                        // for tile j+1's heavy test: its maximum is the shift and lies in this half
                        one_pend[rb] = (need[rb] && hmx == m) ? 1.f : 0.f;
                    }
                    need_any = need_any || need[rb];
                }
                rescale_pend = __builtin_amdgcn_ballot_w64(need_any) != 0;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const float m_new = need[rb] ? m_tile[rb] : m_run[rb];
                    const float alpha = need[rb] ? fast_exp2(m_run[rb] - m_new) : 1.f;
                    m_run[rb] = m_new;
                    l_run[rb] *= alpha;
                    alpha_pend[rb] = alpha;
                    // reuse: the shift for the fma slots.  In masked tiles it is kept finite (a
                    // row with no visible key yet has m = -inf), so that with the positive
                    // multiplier c_mask a hidden score -inf stays -inf through the fma.
                    mx[rb][0] = (MASKED && m_new == kNegInf) ? 0.f : -m_new;
                }
            } else {
                constexpr int E = (NE + NFMA - 1) / NFMA;
                const int k0 = (i - HB - 1) * E;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int f = k0 + e;
                        if (f < NE) {
                            const float t = fmaf(s_nxt[rb][f / 16][f % 16], MASKED ? c_mask : a.scale_log2, mx[rb][0]);
                            s_nxt[rb][f / 16][f % 16] = t;
                        }
                    }
            }
            vf = vf1;
            vf1 = vf2;
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (F8) store_v8(vraw, VB_OTHER);   // V_{j+1}: its buffer was last read in j-1
    };

    // One pipeline iteration for tile j (parity PAR = j & 1); on entry the score registers of
    // parity PAR hold the shifted scores of tile j.
    //   loads    K_{j+2} -> K buffer PAR, V_{j+1} -> V buffer !PAR (tiles past N read zeros)
    //   phase A  MFMA S_{j+1} (K buffer !PAR)           || VALU exp / sum / pack of tile j
    //   phase B  MFMA O^T += V_j^T P_j^T (V buffer PAR) || VALU prep of tile j+1
    // MASKED applies the key mask to tile j+1; a tile with no visible key for a row leaves that
    // row's statistics untouched and contributes zero probability.  A wave whose rows see no key
    // of tile j (causal) only helps with the loads and the barrier.
    auto step = [&](auto par_c, auto masked_c, auto split_c, int j) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_c)::value;
        constexpr int KB_THIS = PAR == 0 ? KB0 : KB1;
        constexpr int VB_OTHER = PAR == 0 ? VB1 : VB0;
        if (rescale_pend) {
            rescale_acc();
            rescale_pend = false;
        }
        if (j < n_w) {
            fast_body(par_c, masked_c, split_c, j);
        } else {
            const __amdgpu_buffer_rsrc_t krs_t = tile_rsrc(a.k, kbase, j + 2);
            const __amdgpu_buffer_rsrc_t vrs_t = tile_rsrc(a.v, kbase, j + 1);
            u32x4 vraw[LPW];
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                buffer_load_lds16(krs_t, buf(KB_THIS) + (i * NW + wave) * 1024, koff[i]);
                if constexpr (F8)
                    vraw[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs_t, voff[i], 0, 0));
                else
                    buffer_load_lds16(vrs_t, buf(VB_OTHER) + (i * NW + wave) * 1024, voff[i]);
            }
            if constexpr (F8) store_v8(vraw, VB_OTHER);
        }
        wait_loads();
        __syncthreads();
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using Mk = std::true_type;
    using Pl = std::false_type;
    using NSp = std::false_type;
    // masked steps of a tile with a row that sees fewer than BN keys take the two-term
    // probabilities (SPLITM); that row's few probabilities are not averaged
    using MSp = std::integral_constant<bool, SPLITM>;
    auto mstep = [&](auto par_c, int jj) __attribute__((always_inline)) { step(par_c, Mk{}, MSp{}, jj); };

    // prologue: K_0, K_1, V_0 into their buffers; S_0 and its preparation
    load_tile(std::false_type{}, 0, KB0);
    load_tile(std::false_type{}, 1, KB1);
    load_tile(std::true_type{}, 0, VB0);
    wait_loads();
    __syncthreads();
    if (n_w > 0) {
        compute_s(sA, KB0);
        pattern_s(V0{});
        prep(sA, 0, 0 >= n_plain);
    }
    __syncthreads();   // K buffer 0 is refilled in iteration 0

    // iterations j < jm see an unmasked tile j+1; the rest apply the mask
    int jm = n_plain - 1;
    jm = jm < n_tiles ? jm : n_tiles;
    int j = 0;
    for (; j + 2 <= jm; j += 2) {
        step(P0{}, Pl{}, NSp{}, j);
        step(P1{}, Pl{}, NSp{}, j + 1);
    }
    if (j < jm) {
        step(P0{}, Pl{}, NSp{}, j);
        ++j;
    }
    if ((j & 1) && j < n_tiles) {
        mstep(P1{}, j);
        ++j;
    }
    for (; j + 2 <= n_tiles; j += 2) {
        mstep(P0{}, j);
        mstep(P1{}, j + 1);
    }
    if (j < n_tiles) mstep(P0{}, j);

    // epilogue.  Output register r of block db is O[qrow][32db + 8(r/4) + 4hh + r%4].
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l_tot = xor32_sum(l_run[rb]);
        // packed sequences under the causal mask: a row may see no key at all (bottom-right
        // alignment with more queries than keys); it gets O = 0 and LSE = -inf
        const bool none = VL && CAUSAL && !(l_tot > 0.f);
        // 8-bit inputs: the value descale multiplies the output (the probabilities never see it)
        const float inv_l = none ? 0.f : (DROP ? a.drop_keep_scale : F8 ? a.v_descale : 1.0f) / l_tot;
        if (qrow[rb] >= N) continue;
        if (hh == 0 && a.lse) a.lse[lbase + qrow[rb]] = none ? kNegInf : (m_run[rb] + __log2f(l_tot)) * kLn2;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = 32 * db + 8 * jj + 4 * hh;
                const float o0 = acc[rb][db][4 * jj + 0] * inv_l;
                const float o1 = acc[rb][db][4 * jj + 1] * inv_l;
                const float o2 = acc[rb][db][4 * jj + 2] * inv_l;
                const float o3 = acc[rb][db][4 * jj + 3] * inv_l;
                if (STF32) {
                    *(f32x4*)((float*)a.o + obase + (int64_t)qrow[rb] * ORSE + d0) = f32x4{o0, o1, o2, o3};
                } else {
                    *(u32x2*)((uint16_t*)a.o + obase + (int64_t)qrow[rb] * ORSE + d0) =
                        u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
                }
            }
    }
}

// Runs query tile qt.  Under the causal mask the tile takes the two-term probabilities in its
// masked steps only when one of its rows sees fewer than BN keys (Lk keys in all, key j
// visible to row i iff j <= i + dlt) -- the first tile of a head, in practice -- and the plain
// instantiation otherwise, so the diagonal tiles of the long rows pay nothing.  Without the
// causal mask the only masked tile is the ragged end of the keys, and it always takes them.
template <int D, int BN, int RB, bool CAUSAL, bool PAD, bool OUT_F32, bool VL, int NW = 4, bool DROP = false,
          bool F8 = false, bool STF32 = OUT_F32>
__device__ __forceinline__ void pipe_tile_dispatch(const FwdArgs& a, int bh, int qt, int Lk, int dlt,
                                                   const SeqGeom& sg) {
    constexpr int BM = NW * 32 * RB;
    if constexpr (OUT_F32 || !CAUSAL) {
        pipe_tile<D, BN, RB, CAUSAL, PAD, OUT_F32, VL, true, NW, DROP, F8, STF32>(a, bh, qt, sg);
    } else {
        const bool few = Lk < BN || qt * BM + 1 + dlt < BN;
        if (few) pipe_tile<D, BN, RB, CAUSAL, PAD, OUT_F32, VL, true, NW, DROP, F8, STF32>(a, bh, qt, sg);
        else pipe_tile<D, BN, RB, CAUSAL, PAD, OUT_F32, VL, false, NW, DROP, F8, STF32>(a, bh, qt, sg);
    }
}

// Work item = one query tile, or under the causal mask a pair of tiles (t, n-1-t) with equal
// total work, so all workgroups of a launch finish together.  NW = 4: 128-row tiles, two
// workgroups per CU.  NW = 8: 256-row tiles, one workgroup per CU (still two waves per SIMD),
// which stages each K/V tile into LDS once for 256 rows instead of twice for 128; it pays off
// for long causal d = 128 heads (+2-3 % at N = 8192 and 131072) and loses where the grid is
// small or the sequences short, so the host picks it only there.
// Workgroups per CU the register budget is sized for: the d = 64, bf16-output kernel fits three
// (at most 168 VGPRs, three waves per SIMD), which hides more latency; the others two, or one of
// eight waves.
template <int D, bool OUT_F32, int NW, bool DROP>
constexpr int pipe_wgs_per_cu() { return NW == 8 ? 1 : (D == 64 && !OUT_F32 && !DROP) ? 3 : 2; }

template <int D, int BN, int RB, bool CAUSAL, bool PAD, bool OUT_F32, int NW = 4, bool DROP = false>
__global__ void __launch_bounds__(64 * NW, (pipe_wgs_per_cu<D, OUT_F32, NW, DROP>())) fa_fwd_bf16_pipe_kernel(FwdArgs a) {
    const TilePair tp = pair_of(xcd_remap(blockIdx.x, a.total_wgs), a.n_qtiles, CAUSAL);
    int Lk = a.N;
    if (PAD) {
        const int s = a.seqlens[tp.bh / a.H];
        Lk = s < 0 ? 0 : (s > a.N ? a.N : s);
    }
    pipe_tile_dispatch<D, BN, RB, CAUSAL, PAD, OUT_F32, false, NW, DROP>(a, tp.bh, tp.qt0, Lk, 0, SeqGeom{});
    if (tp.qt1 >= 0) {
        __syncthreads();   // the first tile's LDS buffers are reused
        pipe_tile_dispatch<D, BN, RB, CAUSAL, PAD, OUT_F32, false, NW, DROP>(a, tp.bh, tp.qt1, Lk, 0, SeqGeom{});
    }
}

// FP8 E4M3 inputs ([B, H, N, d] byte tensors, one descale per tensor): the same work items and
// tile body with S on the 8-bit MFMA (64 head dimensions per step) and V widened to bf16 as it
// is staged, so the value product, its precision and everything after it are the bf16 path's.
// The Q and K descales are folded into a.scale / a.scale_log2 by the host; V's into
// a.v_descale.
template <int D, int BN, bool CAUSAL, bool PAD, bool OUT_F32, int NW = 4>
__global__ void __launch_bounds__(64 * NW, NW == 8 ? 1 : 2) fa_fwd_fp8_pipe_kernel(FwdArgs a) {
    const TilePair tp = pair_of(xcd_remap(blockIdx.x, a.total_wgs), a.n_qtiles, CAUSAL);
    int Lk = a.N;
    if (PAD) {
        const int s = a.seqlens[tp.bh / a.H];
        Lk = s < 0 ? 0 : (s > a.N ? a.N : s);
    }
    pipe_tile_dispatch<D, BN, 1, CAUSAL, PAD, OUT_F32, false, NW, false, true>(a, tp.bh, tp.qt0, Lk, 0, SeqGeom{});
    if (tp.qt1 >= 0) {
        __syncthreads();   // the first tile's LDS buffers are reused
        pipe_tile_dispatch<D, BN, 1, CAUSAL, PAD, OUT_F32, false, NW, false, true>(a, tp.bh, tp.qt1, Lk, 0, SeqGeom{});
    }
}

// Packed variable-length sequences ([T, H, d] token-major tensors, per-sequence query and key
// lengths from prefix sums).  The launch covers the longest query sequence; work item `it` of
// (sequence, head) takes tile `it` of the sequence's own n tiles -- or, when the launch pairs
// causal tiles (enough tiles to fill the chip twice over), the pair (n-1-it, it) -- and items
// past the sequence's tiles exit at once.  Unpaired causal tiles run from the last (most keys)
// to the first.
//
// XCD placement: head bh runs on XCD bh % 8 (the dispatcher deals workgroup ids to the XCDs
// round-robin), its work items contiguous there so its tiles share that XCD's L2.  Heads of
// one sequence are thereby spread over all XCDs and every XCD receives the same mix of short
// and long sequences; grouping consecutive heads per XCD, as for equal-length heads, would
// hand whole sequences, and very unequal amounts of work, to single XCDs.
template <int D, int BN, int RB, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(256, 2) fa_fwd_bf16_varlen_kernel(FwdArgs a) {
    constexpr int BM = 128 * RB;
    const bool paired = CAUSAL && a.pair;
    const int per = paired ? (a.n_qtiles + 1) / 2 : a.n_qtiles;
    const HeadItem hi = head_item_xcd(blockIdx.x, a.B * a.H, per);
    if (hi.bh < 0) return;
    const int bh = hi.bh;
    const int it = hi.it;
    const int b = bh / a.H;
    const SeqGeom sg = varlen_geom(a, b, bh - b * a.H, D);
    const int n = (sg.Lq + BM - 1) / BM;
    int qt0, qt1 = -1;
    if (paired) {
        if (it >= (n + 1) / 2) return;
        qt0 = n - 1 - it;
        if (it < qt0) qt1 = it;
    } else {
        if (it >= n) return;
        qt0 = CAUSAL ? n - 1 - it : it;
    }
    pipe_tile_dispatch<D, BN, RB, CAUSAL, true, OUT_F32, true>(a, bh, qt0, sg.Lk, CAUSAL ? sg.dlt : 0, sg);
    if (qt1 >= 0) {
        __syncthreads();
        pipe_tile_dispatch<D, BN, RB, CAUSAL, true, OUT_F32, true>(a, bh, qt1, sg.Lk, CAUSAL ? sg.dlt : 0, sg);
    }
}


// Packed sequences whose tiles alone would leave most of the chip idle (a few long prefill
// chunks, a single long sequence): the keys of every (sequence, head) are split into
// a.n_ranges ranges of a.range_keys keys, and one workgroup runs query tile qt of head bh over
// the keys of range r only -- the same tile code on a shifted key window (key j of the range
// is key r * range_keys + j of the sequence, and the causal offset moves with it).  Each range
// writes its float32 output rows and its log-sum-exp to the caller's workspace; a row that
// sees no key of the range gets O = 0 and LSE = -inf there.  The probabilities follow the
// final output type's precision rule (OUT_F32).  fa_fwd_varlen_merge_kernel then combines the
// ranges with the online update's rescaling.  Work item: query tile it (heaviest first under
// the causal mask) of the pair (head bh, range r), numbered bh * n_ranges + r; the tiles of one
// pair run on one XCD, which reads that range's keys into its L2 once, and the ranges of one
// head spread over the XCDs.
template <int D, int BN, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(256, 2) fa_fwd_bf16_varlen_split_kernel(FwdArgs a) {
    constexpr int BM = 128;
    const int S = a.n_ranges;
    const HeadItem hi = head_item_xcd(blockIdx.x, a.B * a.H * S, a.n_qtiles);
    if (hi.bh < 0) return;
    const int bh = hi.bh / S;
    const int r = hi.bh - bh * S;
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    const int itq = hi.it;
    const SeqGeom sg = varlen_geom(a, b, h, D);
    const int n = (sg.Lq + BM - 1) / BM;
    if (itq >= n) return;
    const int qt = CAUSAL ? n - 1 - itq : itq;
    const int k_lo = r * a.range_keys;
    const int k_hi = sg.Lk < k_lo + a.range_keys ? sg.Lk : k_lo + a.range_keys;
    SeqGeom rg = sg;
    rg.kbase = sg.kbase + (int64_t)k_lo * sg.rse;
    rg.Lk = k_hi > k_lo ? k_hi - k_lo : 0;
    rg.dlt = sg.dlt - k_lo;
    const int64_t slot = ((int64_t)r * a.B + b) * a.H + h;   // (range, sequence, head)
    rg.obase = slot * a.max_q * D;
    rg.orse = D;
    rg.lbase = slot * a.max_q;
    FwdArgs ar = a;
    ar.o = a.ws_o;
    ar.lse = a.ws_lse;
    pipe_tile_dispatch<D, BN, 1, CAUSAL, true, OUT_F32, true, 4, false, false, true>(ar, bh, qt, rg.Lk, CAUSAL ? rg.dlt : 0, rg);
}

// Combines the key ranges of fa_fwd_varlen_split_kernel: for row i of sequence b, head h,
// LSE = ln sum_r exp(LSE_r) and O = sum_r exp(LSE_r - LSE) O_r, the ranges taken in order (so
// the result is the same on every run).  A row that sees no key at all keeps O = 0 and
// LSE = -inf.  One thread per four columns of a row; rows past a sequence's length are skipped.
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(256) fa_fwd_varlen_merge_kernel(FwdArgs a) {
    constexpr int TPR = D / 4;                       // threads per row
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row_id = gid / TPR;                // ((b * H + h) * max_q + i)
    const int c = (int)(gid % TPR);
    const int i = (int)(row_id % a.max_q);
    const int64_t bh = row_id / a.max_q;
    if (bh >= (int64_t)a.B * a.H) return;
    const int b = (int)(bh / a.H);
    const int h = (int)(bh - (int64_t)b * a.H);
    const SeqGeom sg = varlen_geom(a, b, h, D);
    if (i >= sg.Lq) return;
    const int S = a.n_ranges;
    const int64_t rstride = (int64_t)a.B * a.H * a.max_q;   // rows between consecutive ranges
    float m = kNegInf;
    for (int r = 0; r < S; ++r) m = fmaxf(m, a.ws_lse[r * rstride + row_id]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lse = kNegInf;
    if (m != kNegInf) {
        float wsum = 0.f;
        for (int r = 0; r < S; ++r) {
            const float lr = a.ws_lse[r * rstride + row_id];
            const float w = lr == kNegInf ? 0.f : fast_exp2((lr - m) * 1.4426950408889634f);
            wsum += w;
            const f32x4 x = *(const f32x4*)(a.ws_o + (r * rstride + row_id) * D + 4 * c);
            o += w * x;
        }
        o *= 1.f / wsum;
        lse = m + __logf(wsum);
    }
    const int64_t off = sg.obase + (int64_t)i * sg.orse + 4 * c;
    if (OUT_F32) *(f32x4*)((float*)a.o + off) = o;
    else *(u32x2*)((uint16_t*)a.o + off) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    if (c == 0 && a.lse) a.lse[sg.lbase + i] = lse;
}

}  // namespace fa
