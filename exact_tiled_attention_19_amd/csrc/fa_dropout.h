// Dropout random numbers for the attention kernels: Philox4x32-10 (Salmon, Moraes, Dror and
// Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC '11) and the element mapping of the
// library's dropout contract.
//
// Contract (include/fa.h, fa_fwd_dropout): element (b, h, i, j) -- query row i, key j of head
// bh = b * H + h -- takes byte 4 (i mod 4) + (j mod 4) of the 16 output bytes (little-endian
// words) of the counter (j / 4, i / 4, bh, offset) under the key (seed_lo, seed_hi), and is kept
// iff that byte >= t = round(256 p).  Kept probabilities are scaled by 256 / (256 - t).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_bf16.h"

namespace fa {

// One Philox4x32 block: ten rounds of two 32 x 32 -> 64-bit products (v_mad_u64_u32) and
// three-input xors, the key bumped by the Weyl constants between rounds (scalar adds).
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return u32x4{c0, c1, c2, c3};
}

// Value of x in lane SRC of this lane's quad (DPP quad_perm [SRC, SRC, SRC, SRC]).
template <int SRC>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
    constexpr int CTRL = SRC | (SRC << 2) | (SRC << 4) | (SRC << 6);
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}

// Dropout words of one 32-key half (fk) of a 64-key tile in the forward's S^T layout.  The
// lane owns query row `row` (row mod 4 = its position a in the quad of lanes holding rows
// 4m .. 4m+3) and keys 32 fk + 8 q + 4 hh + 0..3 of the tile (q in 0..3); group q needs word a
// of the Philox block (j4 = kv0 / 4 + 8 fk + 2 q + hh, i4 = row / 4).  The four lanes of a quad
// need the same four blocks, so lane a computes block q = a and the quad exchanges words:
// out[q] = word a of block q.
__device__ __forceinline__ void dropout_words_fwd(uint32_t (&out)[4], int kv0, int fk, int row, int hh, int bh,
                                                  uint32_t offset, uint32_t k0, uint32_t k1) {
    const int a = row & 3;
    const u32x4 w = philox4x32_10(((uint32_t)kv0 >> 2) + 8 * fk + 2 * a + hh, (uint32_t)row >> 2, (uint32_t)bh,
                                  offset, k0, k1);
    auto pick = [&](uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) __attribute__((always_inline)) {
        return a == 0 ? b0 : a == 1 ? b1 : a == 2 ? b2 : b3;
    };
    // block q lives in lane q of the quad
    out[0] = pick(quad_bcast<0>(w[0]), quad_bcast<0>(w[1]), quad_bcast<0>(w[2]), quad_bcast<0>(w[3]));
    out[1] = pick(quad_bcast<1>(w[0]), quad_bcast<1>(w[1]), quad_bcast<1>(w[2]), quad_bcast<1>(w[3]));
    out[2] = pick(quad_bcast<2>(w[0]), quad_bcast<2>(w[1]), quad_bcast<2>(w[2]), quad_bcast<2>(w[3]));
    out[3] = pick(quad_bcast<3>(w[0]), quad_bcast<3>(w[1]), quad_bcast<3>(w[2]), quad_bcast<3>(w[3]));
}

// Keep bits of one 32-row half of a dK/dV tile, key-major layout: the lane owns key `key`
// (key mod 4 = its position a in the quad of lanes holding keys 4m .. 4m+3) and rows
// rbase + 8 q + 4 hh + u (q, u in 0..3).  Rows rbase + 8 q + 4 hh .. +3 form block (key / 4,
// (rbase + 8 q + 4 hh) / 4), whose word u holds row u and whose byte a holds this key; the quad
// needs the same four blocks, so lane a computes block q = a and the quad exchanges the words.
// Bit 4 q + u of the result: is (row rbase + 8 q + 4 hh + u, key) kept?
__device__ __forceinline__ uint32_t dropout_bits_kmajor(int key, int rbase, int hh, int bh, uint32_t offset,
                                                        uint32_t k0, uint32_t k1, uint32_t t) {
    const int a = key & 3;
    const u32x4 w = philox4x32_10((uint32_t)key >> 2, (uint32_t)(rbase + 8 * a + 4 * hh) >> 2, (uint32_t)bh, offset,
                                  k0, k1);
    uint32_t bits = 0;
    auto add = [&](uint32_t x, int bit) __attribute__((always_inline)) {
        bits |= (((x >> (8 * a)) & 0xFFu) >= t ? 1u : 0u) << bit;
    };
#define FA_DROP_KM(Q)                        \
    add(quad_bcast<Q>(w[0]), 4 * (Q) + 0);   \
    add(quad_bcast<Q>(w[1]), 4 * (Q) + 1);   \
    add(quad_bcast<Q>(w[2]), 4 * (Q) + 2);   \
    add(quad_bcast<Q>(w[3]), 4 * (Q) + 3);
    FA_DROP_KM(0)
    FA_DROP_KM(1)
    FA_DROP_KM(2)
    FA_DROP_KM(3)
#undef FA_DROP_KM
    return bits;
}

// Is byte b of word w at least the threshold (element kept)?
__device__ __forceinline__ bool drop_keep(uint32_t w, int b, uint32_t t) { return ((w >> (8 * b)) & 0xFFu) >= t; }

}  // namespace fa
