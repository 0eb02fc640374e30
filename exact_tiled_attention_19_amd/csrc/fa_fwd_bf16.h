// Fused exact-attention forward for bf16 inputs on gfx950 (MI355X).
//
// What is computed: for one (batch, head) and one query row i,
//     O_i = sum_j softmax_j(scale * q_i . k_j over visible keys) v_j,
//     LSE_i = ln sum_j exp(scale * q_i . k_j)
// ("FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical Stability",
// section "What is FlashAttention exact about?").  The keys are consumed one tile at a time
// with the running-statistics update of the same page's section "How can softmax be computed
// across tiles?": a running maximum m, a running sum l of shifted exponentials and an
// unnormalised accumulator, both rescaled by exp(m_old - m_new) when a tile raises the
// maximum; the output is accumulator / l at the end.  Exponentials are taken base 2 on
// scores pre-multiplied by scale*log2(e), which is the same function.
//
// Mapping onto the chip (one workgroup per (batch, head, 128-row query tile), 4 wave64s,
// each wave owns 32 query rows):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with K as the A operand (read from LDS) and
//     Q^T as the B operand (held in VGPRs for the whole kernel).  In the 32x32 accumulator a
//     lane owns one query column and 16 of the 32 keys, so every per-row statistic is
//     reduced inside the lane, plus one exchange with lane^32 for the row maximum.
//   * O^T += V^T P^T on the same instruction: the probabilities come straight out of the S^T
//     accumulator registers as the B operand (no shuffle), V^T is the A operand read from LDS.
//     The row rescale factor is then a per-lane scalar.
//   * K/V tiles are double-buffered in LDS: the global loads of tile t+1 are issued before the
//     MFMAs of tile t and written to the other LDS buffer after them; one barrier per tile.
//   * Masks are applied only on tiles that need them (the causal diagonal, the last tile of a
//     padded or ragged key range) by selecting -inf; tiles entirely above a wave's rows are
//     skipped by that wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_sched.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* seqlens;
    int B, H, N;
    int n_qtiles;      // ceil(N / BM)  (packed sequences: ceil(max_q / BM))
    int total_wgs;     // B * H * work items per head
    float scale;       // multiplier of the raw dot products
    float scale_log2;  // scale * log2(e)
    // packed variable-length sequences only (token-major [T, H, d] tensors)
    const int32_t* cu_q;   // [B + 1] prefix sums of the query lengths
    const int32_t* cu_k;   // [B + 1] prefix sums of the key lengths
    int total_q, total_k;  // tokens in the packed query and key tensors
    int max_q, max_k;      // longest query / key sequence the launch was sized for
    int bottom_right;      // causal alignment: 1 bottom-right, 0 top-left
    int pair;              // causal: a work item is a tile pair (t, n-1-t) of one sequence
    // dropout on the probabilities (kernels instantiated with dropout only)
    uint32_t drop_k0, drop_k1;   // Philox key: the seed's low and high words
    uint32_t drop_offset;        // fourth Philox counter word
    uint32_t drop_t;             // byte threshold round(256 p): kept iff byte >= drop_t
    float drop_keep_scale;       // 256 / (256 - drop_t)
    // 8-bit inputs only: the value tensor's descale, applied to the output
    float v_descale;
    // packed sequences with the keys split into ranges (split tile kernel and its merge): the
    // caller's workspace holds every range's float32 output rows and log-sum-exps
    float* ws_o;           // [n_ranges][B][H][max_q][d]
    float* ws_lse;         // [n_ranges][B][H][max_q]
    int n_ranges;          // key ranges per (sequence, head)
    int range_keys;        // keys per range (a multiple of the key tile)
};

using FwdKernelFn = void (*)(FwdArgs);

// The forward kernel for FP8 E4M3 inputs (fa_fp8.hip) for head width d, mask bits `mask` and
// output type; `wide` asks for the eight-wave 256-row workgroup where one exists, `small` for
// the key-split kernel of small grids.  Sets the query rows per tile (*bm) and threads per
// workgroup; nullptr when d has no kernel.
__attribute__((visibility("hidden"))) FwdKernelFn pick_fp8_kernel(int d, int mask, bool out_f32, bool wide, bool small,
                                                                  int* bm, int* threads);

// Where the rows of one head of one sequence live, and which keys its queries may see.
struct SeqGeom {
    int64_t qbase;  // element offset of query row 0
    int64_t kbase;  // element offset of key (and value) row 0
    int64_t lbase;  // index of row 0's log-sum-exp
    int64_t obase;  // element offset of output row 0
    int Lq;         // query rows
    int Lk;         // keys
    int dlt;        // causal mask: key j is visible to query row i iff j <= i + dlt
    int rse;        // elements between consecutive input rows
    int orse;       // elements between consecutive output rows
};

// Sequence b, head h of a packed batch.  Offsets are clamped into the tensors, so any
// cu_seqlens values stay memory-safe; lengths are capped at the sizes the launch covers.
// Bottom-right alignment places the Lq queries at the last Lq of the Lk key positions.
__device__ __forceinline__ SeqGeom varlen_geom(const FwdArgs& a, int b, int h, int D) {
    auto clampi = [](int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); };
    const int qs = clampi(a.cu_q[b], 0, a.total_q);
    const int qe = clampi(a.cu_q[b + 1], qs, a.total_q);
    const int ks = clampi(a.cu_k[b], 0, a.total_k);
    const int ke = clampi(a.cu_k[b + 1], ks, a.total_k);
    SeqGeom g;
    g.Lq = qe - qs < a.max_q ? qe - qs : a.max_q;
    g.Lk = ke - ks < a.max_k ? ke - ks : a.max_k;
    g.dlt = a.bottom_right ? g.Lk - g.Lq : 0;
    g.rse = a.H * D;
    g.qbase = ((int64_t)qs * a.H + h) * D;
    g.kbase = ((int64_t)ks * a.H + h) * D;
    g.lbase = (int64_t)h * a.total_q + qs;
    g.obase = g.qbase;
    g.orse = g.rse;
    return g;
}

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the two lane halves (lane l and lane l^32).  v_permlane32_swap with the
// same register as both operands leaves the lower half's values in the first result and the
// upper half's in the second, on every lane.
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Kernel variants (same result, different instruction choices):
//   VT = 0: V^T operand gathered with eight 16-bit LDS reads per fragment.
//   VT = 1: V^T operand read with ds_read_b64_tr_b16 (LDS transpose read), two per fragment.
template <int D, int BN, bool CAUSAL, bool PAD, bool OUT_F32, int VT>
__global__ void __launch_bounds__(256, 2) fa_fwd_bf16_kernel(FwdArgs a) {
    constexpr int BM = 128;                 // query rows per workgroup
    constexpr int NT = 256;                 // threads per workgroup
    constexpr int KC = D / 16;              // k-steps of the S MFMA (16 of d each)
    constexpr int NKB = BN / 32;            // 32-key blocks per tile
    constexpr int NDB = D / 32;             // 32-wide blocks of d in the output
    constexpr int PC = BN / 16;             // k-steps of the PV MFMA (16 keys each)
    constexpr int KSTR = D + 8;             // K row stride in LDS (elements): 16-byte pad
    constexpr int VSTR = D + 32;            // V row stride in LDS (elements): 64-byte pad
    constexpr int KBUF = BN * KSTR;
    constexpr int VBUF = BN * VSTR;
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int LDC = BN * CPR / NT;      // 16-byte chunks per thread per tensor per tile
    constexpr bool PRECISE = OUT_F32;       // split P into two bf16 terms for fp32 output
    static_assert(LDC * NT == BN * CPR, "tile must split evenly over the workgroup");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KBUF + 2 * VBUF];
    uint16_t* const kbuf = smem;
    uint16_t* const vbuf = smem + 2 * KBUF;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const TileCoord tc = tile_of(xcd_remap(blockIdx.x, a.total_wgs), a.n_qtiles, CAUSAL);
    const int b = tc.bh / a.H;
    const int N = a.N;
    const int q0 = tc.qt * BM;
    const int qw0 = q0 + wave * 32;         // first query row of this wave
    const int qrow = qw0 + l32;             // the query row this lane's statistics belong to
    const int64_t base = (int64_t)tc.bh * N * D;

    int Lk = N;                             // keys [0, Lk) exist for this batch element
    if (PAD) {
        const int s = a.seqlens[b];
        Lk = s < 0 ? 0 : (s > N ? N : s);
    }

    if (Lk == 0) {  // every key masked: O = 0, LSE = -inf (defined all-masked convention)
        if (qrow < N) {
            if (hh == 0 && a.lse) a.lse[(int64_t)tc.bh * N + qrow] = kNegInf;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = 32 * db + 8 * j + 4 * hh;
                    if (OUT_F32) {
                        float* op = (float*)a.o + base + (int64_t)qrow * D + d0;
                        *(f32x4*)op = f32x4{0.f, 0.f, 0.f, 0.f};
                    } else {
                        uint16_t* op = (uint16_t*)a.o + base + (int64_t)qrow * D + d0;
                        *(u32x2*)op = u32x2{0u, 0u};
                    }
                }
        }
        return;
    }

    int kv_end = Lk;
    if (CAUSAL) kv_end = kv_end < q0 + BM ? kv_end : q0 + BM;
    const int n_tiles = (kv_end + BN - 1) / BN;

    // this lane's slice of Q^T as MFMA B operands: Q[qrow][16c + 8hh .. +8].
    bf16x8 qf[KC];
    {
        const uint16_t* qp = (const uint16_t*)a.q + base + (int64_t)(qrow < N ? qrow : N - 1) * D + 8 * hh;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            qf[c] = *(const bf16x8*)(qp + 16 * c);
            if (qrow >= N) qf[c] = bf16x8{};
        }
    }

    // K/V tile staging.  Chunk ci of a tile is 16 bytes at row ci / CPR, column chunk
    // ci % CPR; consecutive threads take consecutive chunks, so each wave reads whole rows.
    const uint16_t* const kg = (const uint16_t*)a.k + base;
    const uint16_t* const vg = (const uint16_t*)a.v + base;
    u32x4 kr[LDC], vr[LDC];
    auto gload = [&](int tile) {
        const int kv0 = tile * BN;
#pragma unroll
        for (int i = 0; i < LDC; ++i) {
            const int ci = tid + NT * i;
            const int row = ci / CPR;
            const int cc = ci - row * CPR;
            int gr = kv0 + row;
            gr = gr < N ? gr : N - 1;   // rows past N are read from row N-1 and masked
            kr[i] = *(const u32x4*)(kg + (int64_t)gr * D + cc * 8);
            vr[i] = *(const u32x4*)(vg + (int64_t)gr * D + cc * 8);
        }
    };
    auto swrite = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LDC; ++i) {
            const int ci = tid + NT * i;
            const int row = ci / CPR;
            const int cc = ci - row * CPR;
            *(u32x4*)(kbuf + buf * KBUF + row * KSTR + cc * 8) = kr[i];
            *(u32x4*)(vbuf + buf * VBUF + row * VSTR + cc * 8) = vr[i];
        }
    };

    // V^T operand for key chunk pc (16 keys) and output block db: lane (d = 32db + l32, hh)
    // holds V[16pc + kmap(hh, e)][d], e = 0..7, kmap(h, e) = 8(e/4) + 4h + e%4 -- the same key
    // order in which the S^T accumulator hands this lane its probabilities.
    auto vt_frag = [&](const uint16_t* vs, int pc, int db) -> bf16x8 {
        if constexpr (VT == 0) {
            uint16_t e16[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = 16 * pc + 8 * (e >> 2) + 4 * hh + (e & 3);
                e16[e] = vs[key * VSTR + 32 * db + l32];
            }
            bf16x8 r;
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] = __builtin_bit_cast(__bf16, e16[e]);
            return r;
        } else {
            // ds_read_b64_tr_b16 works on groups of 16 lanes: lane j of a group supplies the
            // address of 4 consecutive 16-bit elements (row j/4, column chunk j%4 of a 4 x 16
            // block) and receives column j of that block, one element per row.  Here a group
            // covers 16 consecutive d and the 4 keys 16pc + 4hh + 0..3 (second read: +8).
            const int row = 16 * pc + 4 * hh + ((l32 & 15) >> 2);
            const int col = 32 * db + (l32 & 16) + 4 * (l32 & 3);
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            // whole-register reinterpretation only: rebuilding the vector element by element
            // through 16-bit casts was observed to miscompile into duplicated dwords
            const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vs + row * VSTR + col)));
            const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vs + (row + 8) * VSTR + col)));
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            const bf16x8 r = __builtin_bit_cast(bf16x8, w);
            return r;
        }
    };

    float m_run = kNegInf;   // running maximum of scale*log2(e)*s over visible keys
    float l_run = 0.f;       // this lane's half of the running sum of 2^(.. - m_run)
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
        const uint16_t* ks = kbuf + (t & 1) * KBUF;
        const uint16_t* vs = vbuf + (t & 1) * VBUF;
        // a tile entirely above this wave's rows carries no visible key for any of them
        const bool wave_active = !CAUSAL || kv0 <= qw0 + 31;
        if (wave_active) {
            // S^T block kb: rows = keys kv0 + 32kb + .., columns = this wave's 32 queries
            f32x16 s[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                s[kb] = f32x16{};
#pragma unroll
                for (int c = 0; c < KC; ++c) {
                    const bf16x8 kf = *(const bf16x8*)(ks + (32 * kb + l32) * KSTR + 16 * c + 8 * hh);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
                }
            }
            // mask -- accumulator register r of block kb holds key kv0+32kb+8(r/4)+4hh+r%4
            const bool need_mask = (kv0 + BN > Lk) || (CAUSAL && kv0 + BN - 1 > qw0);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                        const bool ok = key < Lk && (!CAUSAL || key <= qrow);
                        s[kb][r] = ok ? s[kb][r] : kNegInf;
                    }
            }
            // online statistics
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = xor32_max(mx);
            const float m_tile = (mx == kNegInf) ? kNegInf : mx * a.scale_log2;
            const float m_new = fmaxf(m_run, m_tile);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(s[kb][r], a.scale_log2, -m_use));
                    s[kb][r] = p;
                }
            if (need_mask) {  // exact zeros for masked keys also when scale == 0
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                        const bool ok = key < Lk && (!CAUSAL || key <= qrow);
                        s[kb][r] = ok ? s[kb][r] : 0.f;
                    }
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) rs += s[kb][r];
            l_run = alpha * l_run + rs;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;

            // O^T += V^T P^T.  Key chunk pc = registers 8(pc%2) .. +7 of block pc/2.
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) {
                const int kb = pc >> 1;
                const int r0 = 8 * (pc & 1);
                u32x4 ph;
#pragma unroll
                for (int e = 0; e < 4; ++e) ph[e] = pack_bf16x2(s[kb][r0 + 2 * e], s[kb][r0 + 2 * e + 1]);
                const bf16x8 phi = __builtin_bit_cast(bf16x8, ph);
                bf16x8 plo;
                if constexpr (PRECISE) {
                    u32x4 pl;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pl[e] = pack_bf16x2(s[kb][r0 + 2 * e] - bf16_lo_to_f32(ph[e]),
                                            s[kb][r0 + 2 * e + 1] - bf16_hi_to_f32(ph[e]));
                    plo = __builtin_bit_cast(bf16x8, pl);
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 vf = vt_frag(vs, pc, db);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, phi, acc[db], 0, 0, 0);
                    if constexpr (PRECISE)
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, plo, acc[db], 0, 0, 0);
                }
            }
        }
        if (has_next) swrite((t + 1) & 1);
        __syncthreads();
    }

    // epilogue.  Output register r of block db is O[qrow][32db + 8(r/4) + 4hh + r%4].
    const float l_tot = xor32_sum(l_run);
    const float inv_l = 1.0f / l_tot;
    if (qrow < N) {
        if (hh == 0 && a.lse) a.lse[(int64_t)tc.bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 32 * db + 8 * j + 4 * hh;
                const float o0 = acc[db][4 * j + 0] * inv_l;
                const float o1 = acc[db][4 * j + 1] * inv_l;
                const float o2 = acc[db][4 * j + 2] * inv_l;
                const float o3 = acc[db][4 * j + 3] * inv_l;
                if (OUT_F32) {
                    float* op = (float*)a.o + base + (int64_t)qrow * D + d0;
                    *(f32x4*)op = f32x4{o0, o1, o2, o3};
                } else {
                    uint16_t* op = (uint16_t*)a.o + base + (int64_t)qrow * D + d0;
                    *(u32x2*)op = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
                }
            }
    }
}

}  // namespace fa
