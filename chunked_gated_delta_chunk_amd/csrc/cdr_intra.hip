// Intra-chunk kernel: everything about one chunk of one head that does not depend on the
// state carried between chunks.  Follows sections M1-M3 of the page
// "PyPTO-Gym 的 chunk_kda 算子实战" (gate prefix sum, decayed A with its triangular
// inverse, the w / u projections) plus the chunk-local factors that section M4 consumes.
//
// One workgroup (4 waves) per (chunk slot, head).  Phases:
//   E    every thread owns a 16-row x 4-column block of the chunk (one 16-row tile) and
//        issues all of its loads (g, k, q, v) at once.  gamma = prefix sum of g inside the
//        tile, plus the totals of the tiles above (through LDS).  Per-element decay
//        factors relative to the tile's middle row m, and the element-wise outputs: qg,
//        kg^T (split), exp(gamma_C), (exp(gamma) k)^T (split, scratch) and v^T (scratch).
//   AA2  16x16 tiles of A (strictly lower, times beta) and A2 (lower incl. diagonal,
//        times scale) on bf16 MFMA.  Per-dimension gates enter the operands through
//        the tile pivots: for rows i in tile R and columns j in tile J <= R,
//          exp(g_i - g_j) = [exp(g_i - g_m(R)) exp(g_m(R) - g_m(J))] * exp(g_m(J) - g_j)
//        so no factor exceeds exp(half a tile's gate span) and the product never
//        overflows.  A uses hi/lo split operands (three MFMAs); A2 feeds only the output
//        and uses single bf16 operands.  Per-head gates use raw q, k (exact bf16
//        products) and apply the scalar decay afterwards.  Wave w owns tile rows w and
//        NT-1-w, which balances the triangle.
//   INV  T = (I + A)^-1 by block-triangular inversion: the 16x16 diagonal blocks by
//        forward substitution in fp32, then blocks are merged 16->32->64->128 with
//        T21 = -T22 (A21 T11), two tile-parallel steps per level on split-bf16 MFMAs.
//   WU   w = T diag(beta) (exp(gamma) k) and u = T diag(beta) v on split-bf16 MFMAs; the
//        right-hand-side fragments are fetched right after phase E.
#include "cdr_common.h"

namespace cdr {

template <int C>
struct IntraShape {
    static constexpr int NT = C / 16;                  // 16-row tiles per chunk
    static constexpr int NPAIR = NT * (NT + 1) / 2;    // lower tiles incl. diagonal
    static constexpr int NOFF = NT * (NT - 1) / 2;     // strictly lower tiles
    static constexpr int SMAX = NT + 1;                // tiles per wave in phase AA2
    static constexpr int EP_LD = KD + 4;               // padded row stride (floats)
    static constexpr int COL_LD = KD + 8;              // padded row stride (bf16)
    static constexpr int TILE_LD = 20;                 // padded 16x16 tile row stride
    static constexpr int TILE_SZ = 16 * TILE_LD;
    static constexpr int NS = C / 32;                  // 32-wide steps along the chunk
    // LDS regions (bytes)
    static constexpr int R1 = C * EP_LD * 4;           // Ep; later A tiles and merge scratch
    static constexpr int R2 = 2 * C * COL_LD * 2;      // column operands; later T tiles
    static constexpr int RF = (NOFF > NT ? NOFF : NT) * KD * 4;  // tile totals, later F
    static constexpr int RG = 2 * NT * KD * 4;         // gamma and exp(gamma) at tile middles
    static constexpr int RMISC = 2 * C * 4;            // beta, per-head gamma
    static constexpr int BYTES = R1 + R2 + RF + RG + RMISC;
    static_assert((NPAIR + (NT / 2) * (NT / 2)) * TILE_SZ * 4 <= R1, "A tiles + merge scratch");
    static_assert(NPAIR * TILE_SZ * 4 <= R2, "T tiles");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int tri(int R, int J) { return R * (R + 1) / 2 + J; }  // J <= R

// 16x16x16 split-bf16 product accumulate: acc += A_tile(fp32, LDS, row-major) * B_tile(fp32, LDS)
__device__ __forceinline__ void tile_mma(f32x4& acc, const float* At, const float* Bt, int r16, int q4, int ld) {
    const float4 av = *reinterpret_cast<const float4*>(At + r16 * ld + 4 * q4);
    const float aa[4] = {av.x, av.y, av.z, av.w};
    const float bb[4] = {Bt[(4 * q4 + 0) * ld + r16], Bt[(4 * q4 + 1) * ld + r16], Bt[(4 * q4 + 2) * ld + r16],
                         Bt[(4 * q4 + 3) * ld + r16]};
    bf16x4 ah, al, bh, bl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        short x, y;
        split_bf(aa[e], x, y); ah[e] = x; al[e] = y;
        split_bf(bb[e], x, y); bh[e] = x; bl[e] = y;
    }
    acc = mfma16(ah, bh, acc);
    acc = mfma16(al, bh, acc);
    acc = mfma16(ah, bl, acc);
}

__device__ __forceinline__ void tile_store(float* Tt, const f32x4& v, float sgn, int r16, int q4, int ld) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) Tt[(4 * q4 + rr) * ld + r16] = sgn * v[rr];
}

template <int C, bool PER_DIM>
__global__ __launch_bounds__(NTHREADS) void intra_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, ChunkMap map, int H, float scale,
    Work ws) {
    using S = IntraShape<C>;
    constexpr int NT = S::NT, NS = S::NS;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::BYTES];
    float* Ep = reinterpret_cast<float*>(smem);                                   // [C][EP_LD]
    uint16_t* colh = reinterpret_cast<uint16_t*>(smem + S::R1);                   // [C][COL_LD]
    uint16_t* coll = colh + C * S::COL_LD;
    float* F = reinterpret_cast<float*>(smem + S::R1 + S::R2);                   // [NOFF][KD]
    float* ttot = F;                                                              // [NT][KD], before F
    float* gmid = reinterpret_cast<float*>(smem + S::R1 + S::R2 + S::RF);        // [NT][KD]
    float* egm = gmid + NT * KD;                                                  // [NT][KD]
    float* bet = egm + NT * KD;                                                   // [C]
    float* grow = bet + C;                                                        // [C] per-head gamma
    float* Atile = reinterpret_cast<float*>(smem);                                // after AA2
    float* Pscr = Atile + S::NPAIR * S::TILE_SZ;                                  // merge scratch
    float* Ttile = reinterpret_cast<float*>(smem + S::R1);

    const int slot = blockIdx.x, h = blockIdx.y;
    int64_t tok0;
    int rows;
    slot_chunk(map, slot, tok0, rows);
    if (rows == 0) return;
    const size_t ch = (size_t)slot * H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const size_t rs = (size_t)H * KD;  // token stride of q, k, v, per-dim g (elements)
    const size_t base = (size_t)tok0 * rs + (size_t)h * KD;

    // ------------------------------------------------------------------ phase E
    {
        const int R = tid >> 5, d0 = 4 * (tid & 31);  // tile row R, columns d0..d0+3
        const bool act = R < NT;
        float gm4[16][4];
        uint2 kr[16], vr[16];
        if (tid < C) {
            const float bv = beta[(size_t)(tok0 + min(tid, rows - 1)) * H + h];
            bet[tid] = (tid < rows) ? bv : 0.f;
        }
        if (act) {
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                // rows past the end of the sequence read its last row and are zeroed: the
                // loads stay unconditional and can all be in flight together
                const int i = 16 * R + ii, ic = min(i, rows - 1);
                const bool ok = i < rows;
                float4 gv;
                if constexpr (PER_DIM) {
                    gv = *reinterpret_cast<const float4*>(g + base + (size_t)ic * rs + d0);
                } else {
                    const float s1 = g[(size_t)(tok0 + ic) * H + h];
                    gv = make_float4(s1, s1, s1, s1);
                }
                const uint2 kx = *reinterpret_cast<const uint2*>(k + base + (size_t)ic * rs + d0);
                const uint2 vx = *reinterpret_cast<const uint2*>(v + base + (size_t)ic * rs + d0);
                kr[ii] = ok ? kx : make_uint2(0, 0);
                vr[ii] = ok ? vx : make_uint2(0, 0);
                gm4[ii][0] = ok ? gv.x : 0.f; gm4[ii][1] = ok ? gv.y : 0.f;
                gm4[ii][2] = ok ? gv.z : 0.f; gm4[ii][3] = ok ? gv.w : 0.f;
            }
#pragma unroll
            for (int ii = 1; ii < 16; ++ii)
#pragma unroll
                for (int c = 0; c < 4; ++c) gm4[ii][c] += gm4[ii - 1][c];
            *reinterpret_cast<float4*>(ttot + R * KD + d0) = make_float4(gm4[15][0], gm4[15][1], gm4[15][2], gm4[15][3]);
        }
        lds_barrier();
        if (act) {
            float off[4] = {0.f, 0.f, 0.f, 0.f}, gcl[4] = {0.f, 0.f, 0.f, 0.f};
            for (int Rp = 0; Rp < NT; ++Rp) {
                const float4 t = *reinterpret_cast<const float4*>(ttot + Rp * KD + d0);
                const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (Rp < R) off[c] += tv[c];
                    gcl[c] += tv[c];
                }
            }
#pragma unroll
            for (int ii = 0; ii < 16; ++ii)
#pragma unroll
                for (int c = 0; c < 4; ++c) gm4[ii][c] += off[c];
            float gmv[4], e_gm[4], e_cm[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                gmv[c] = gm4[8][c];
                e_gm[c] = ex(gmv[c]);            // exp(gamma_m)
                e_cm[c] = ex(gcl[c] - gmv[c]);   // exp(gamma_C - gamma_m) <= 1
            }
            *reinterpret_cast<float4*>(gmid + R * KD + d0) = make_float4(gmv[0], gmv[1], gmv[2], gmv[3]);
            *reinterpret_cast<float4*>(egm + R * KD + d0) = make_float4(e_gm[0], e_gm[1], e_gm[2], e_gm[3]);
            if (R == 0)
                *reinterpret_cast<float4*>(ws.gC + ch * KD + d0) =
                    make_float4(ex(gcl[0]), ex(gcl[1]), ex(gcl[2]), ex(gcl[3]));
            if constexpr (!PER_DIM) {
                if ((tid & 31) == 0) {
#pragma unroll
                    for (int ii = 0; ii < 16; ++ii) grow[16 * R + ii] = gm4[ii][0];
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                // transposed outputs of rows 16R + 8hh .. +7, packed two bf16 per register
                uint32_t bwh[4][4], bwl[4][4], kgh[4][4], kgl[4][4], vtp[4][4];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ii = 8 * hh + e, i = 16 * R + ii;
                    float kf[4], ep[4];
                    kf[0] = __uint_as_float(kr[ii].x << 16); kf[1] = __uint_as_float(kr[ii].x & 0xffff0000u);
                    kf[2] = __uint_as_float(kr[ii].y << 16); kf[3] = __uint_as_float(kr[ii].y & 0xffff0000u);
                    const uint32_t vh[4] = {vr[ii].x & 0xffffu, vr[ii].x >> 16, vr[ii].y & 0xffffu, vr[ii].y >> 16};
                    short chs[4], cls[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float x = gm4[ii][c] - gmv[c];
                        ep[c] = ex(x);             // exp(gamma_i - gamma_m)
                        const float em = ex(-x);   // exp(gamma_m - gamma_i)
                        if constexpr (PER_DIM) split_bf(kf[c] * em, chs[c], cls[c]);
                        const float egi = e_gm[c] * ep[c];               // exp(gamma_i)
                        short bh, bl, gh, gl;
                        split_bf(kf[c] * egi, bh, bl);                   // beta enters through T diag(beta)
                        split_bf(kf[c] * (em * e_cm[c]), gh, gl);        // exp(gamma_C - gamma_i) k
                        if ((e & 1) == 0) {
                            bwh[c][e >> 1] = (uint16_t)bh; bwl[c][e >> 1] = (uint16_t)bl;
                            kgh[c][e >> 1] = (uint16_t)gh; kgl[c][e >> 1] = (uint16_t)gl;
                            vtp[c][e >> 1] = vh[c];
                        } else {
                            bwh[c][e >> 1] |= (uint32_t)(uint16_t)bh << 16; bwl[c][e >> 1] |= (uint32_t)(uint16_t)bl << 16;
                            kgh[c][e >> 1] |= (uint32_t)(uint16_t)gh << 16; kgl[c][e >> 1] |= (uint32_t)(uint16_t)gl << 16;
                            vtp[c][e >> 1] |= vh[c] << 16;
                        }
                    }
                    if constexpr (PER_DIM) {
                        *reinterpret_cast<float4*>(Ep + i * S::EP_LD + d0) = make_float4(ep[0], ep[1], ep[2], ep[3]);
                        *reinterpret_cast<uint2*>(colh + i * S::COL_LD + d0) = pack4(chs);
                        *reinterpret_cast<uint2*>(coll + i * S::COL_LD + d0) = pack4(cls);
                    }
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    // (K, C) / (V, C) fragment (d / 16, R / 2): rows 16 R + 8 hh .. +7 of column d
                    // are exactly the 16-byte slot of lane (d % 16) + 16 (2 (R % 2) + hh)
                    const int d = d0 + c;
                    const size_t tcol = ch * KD * C + frag(d >> 4, R >> 1, C / 32) + ((d & 15) + 16 * (2 * (R & 1) + hh)) * 8;
                    *reinterpret_cast<uint4*>(ws.bwT_hi + tcol) = make_uint4(bwh[c][0], bwh[c][1], bwh[c][2], bwh[c][3]);
                    *reinterpret_cast<uint4*>(ws.bwT_lo + tcol) = make_uint4(bwl[c][0], bwl[c][1], bwl[c][2], bwl[c][3]);
                    *reinterpret_cast<uint4*>(ws.kgT_hi + tcol) = make_uint4(kgh[c][0], kgh[c][1], kgh[c][2], kgh[c][3]);
                    *reinterpret_cast<uint4*>(ws.kgT_lo + tcol) = make_uint4(kgl[c][0], kgl[c][1], kgl[c][2], kgl[c][3]);
                    *reinterpret_cast<uint4*>(ws.vT + tcol) = make_uint4(vtp[c][0], vtp[c][1], vtp[c][2], vtp[c][3]);
                }
            }
        }
        lds_barrier();
        if constexpr (PER_DIM) {
            // strictly lower pairs p = R(R-1)/2 + J: F = exp(gamma_m(R) - gamma_m(J)) <= 1
            for (int e = 4 * tid; e < S::NOFF * KD; e += 4 * NTHREADS) {
                const int p = e / KD, d = e % KD;
                const int R = (int)((1.f + __builtin_sqrtf(8.f * p + 1.f)) * 0.5f);  // R(R-1)/2 <= p < R(R+1)/2
                const int J = p - R * (R - 1) / 2;
                const float4 a = *reinterpret_cast<const float4*>(gmid + R * KD + d);
                const float4 b = *reinterpret_cast<const float4*>(gmid + J * KD + d);
                *reinterpret_cast<float4*>(F + e) = make_float4(ex(a.x - b.x), ex(a.y - b.y), ex(a.z - b.z), ex(a.w - b.w));
            }
        }
    }
    lds_barrier();
    // row-operand fragments of phase AA2 (rows w and NT-1-w)
    const bool aa_active = wave < NT / 2;
    const int Rown[2] = {wave, NT - 1 - wave};
    uint4 kfr[2][KD / 32], qfr[2][KD / 32];
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks) {
            const int i = 16 * Rown[o] + r16, ic = min(i, rows - 1);
            const uint4 kx = *reinterpret_cast<const uint4*>(k + base + (size_t)ic * rs + 32 * ks + 8 * q4);
            const uint4 qx = *reinterpret_cast<const uint4*>(q + base + (size_t)ic * rs + 32 * ks + 8 * q4);
            kfr[o][ks] = (i < rows) ? kx : make_uint4(0, 0, 0, 0);
            qfr[o][ks] = (i < rows) ? qx : make_uint4(0, 0, 0, 0);
        }

    // ------------------------------------------------------------------ phase AA2
    f32x4 accA[S::SMAX];
#pragma unroll
    for (int s = 0; s < S::SMAX; ++s) {
        accA[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!aa_active) continue;
        const int o = (s <= wave) ? 0 : 1;          // which owned row
        const int R = Rown[o];
        const int J = (o == 0) ? s : s - wave - 1;
        if (J > R) continue;
        const int i = 16 * R + r16, j = 16 * J + r16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks) {
            const int dd = 32 * ks + 8 * q4;
            const uint4 krv = o ? kfr[1][ks] : kfr[0][ks];
            const uint4 qrv = o ? qfr[1][ks] : qfr[0][ks];
            if constexpr (PER_DIM) {
                float kf[8], qf[8], ep[8];
                unpack8(krv, kf);
                unpack8(qrv, qf);
                const float4* epp = reinterpret_cast<const float4*>(Ep + i * S::EP_LD + dd);
                const float4 e0 = epp[0], e1 = epp[1];
                ep[0] = e0.x; ep[1] = e0.y; ep[2] = e0.z; ep[3] = e0.w;
                ep[4] = e1.x; ep[5] = e1.y; ep[6] = e1.z; ep[7] = e1.w;
                if (J < R) {
                    const float4* fp = reinterpret_cast<const float4*>(F + (R * (R - 1) / 2 + J) * KD + dd);
                    const float4 f0 = fp[0], f1 = fp[1];
                    ep[0] *= f0.x; ep[1] *= f0.y; ep[2] *= f0.z; ep[3] *= f0.w;
                    ep[4] *= f1.x; ep[5] *= f1.y; ep[6] *= f1.z; ep[7] *= f1.w;
                }
                if (J == R) {
                    // qg = scale q exp(gamma) = scale q Ep exp(gamma_m): (C, K) fragment (R, ks)
                    const float4* gp = reinterpret_cast<const float4*>(egm + R * KD + dd);
                    const float4 g0 = gp[0], g1 = gp[1];
                    const float eg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                    uint4 pq;
                    pq.x = pack_bf2(scale * qf[0] * ep[0] * eg[0], scale * qf[1] * ep[1] * eg[1]);
                    pq.y = pack_bf2(scale * qf[2] * ep[2] * eg[2], scale * qf[3] * ep[3] * eg[3]);
                    pq.z = pack_bf2(scale * qf[4] * ep[4] * eg[4], scale * qf[5] * ep[5] * eg[5]);
                    pq.w = pack_bf2(scale * qf[6] * ep[6] * eg[6], scale * qf[7] * ep[7] * eg[7]);
                    *reinterpret_cast<uint4*>(ws.qg + ch * C * KD + frag(R, ks, KD / 32) + lane * 8) = pq;
                }
                bf16x8 ahi, alo, aq;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    short hh, ll;
                    split_bf(kf[e] * ep[e], hh, ll);
                    ahi[e] = hh;
                    alo[e] = ll;
                    aq[e] = (short)f2bf(qf[e] * ep[e]);
                }
                const bf16x8 bhi = as_bf16x8(*reinterpret_cast<const uint4*>(colh + j * S::COL_LD + dd));
                const bf16x8 blo = as_bf16x8(*reinterpret_cast<const uint4*>(coll + j * S::COL_LD + dd));
                acc = mfma32(ahi, bhi, acc);
                acc = mfma32(alo, bhi, acc);
                acc = mfma32(ahi, blo, acc);
                acc2 = mfma32(bhi, aq, acc2);   // A2^T tile: rows j, columns i
            } else {
                const uint4 kx = *reinterpret_cast<const uint4*>(k + base + (size_t)min(j, rows - 1) * rs + dd);
                const bf16x8 b = as_bf16x8((j < rows) ? kx : make_uint4(0, 0, 0, 0));
                if (J == R) {
                    float qf[8];
                    unpack8(qrv, qf);
                    const float f = scale * ex(grow[i]);
                    uint4 pq;
                    pq.x = pack_bf2(f * qf[0], f * qf[1]);
                    pq.y = pack_bf2(f * qf[2], f * qf[3]);
                    pq.z = pack_bf2(f * qf[4], f * qf[5]);
                    pq.w = pack_bf2(f * qf[6], f * qf[7]);
                    *reinterpret_cast<uint4*>(ws.qg + ch * C * KD + frag(R, ks, KD / 32) + lane * 8) = pq;
                }
                acc = mfma32(as_bf16x8(krv), b, acc);
                acc2 = mfma32(b, as_bf16x8(qrv), acc2);   // A2^T tile: rows j, columns i
            }
        }
        // A tile: rows i = 16 R + 4 q4 + rr, column j = 16 J + r16
        // A2^T tile: rows j = 16 J + 4 q4 + rr, column i = 16 R + r16
        float a2v[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int ii = 16 * R + 4 * q4 + rr, jj = 16 * J + r16;
            const int i2 = 16 * R + r16, j2 = 16 * J + 4 * q4 + rr;
            float a = acc[rr], a2 = acc2[rr];
            if constexpr (!PER_DIM) {
                a *= (jj <= ii) ? ex(grow[ii] - grow[jj]) : 0.f;
                a2 *= (j2 <= i2) ? ex(grow[i2] - grow[j2]) : 0.f;
            }
            accA[s][rr] = (jj < ii) ? a * bet[ii] : 0.f;
            a2v[rr] = (j2 <= i2) ? a2 * scale : 0.f;
        }
        *reinterpret_cast<uint2*>(ws.A2 + ch * C * C + frag(R, J >> 1, C / 32) + fragT(J & 1, r16, q4)) =
            make_uint2(pack_bf2(a2v[0], a2v[1]), pack_bf2(a2v[2], a2v[3]));
    }
    lds_barrier();

    // ------------------------------------------------------------------ phase INV
#pragma unroll
    for (int s = 0; s < S::SMAX; ++s) {
        if (!aa_active) continue;
        const int o = (s <= wave) ? 0 : 1;
        const int R = Rown[o];
        const int J = (o == 0) ? s : s - wave - 1;
        if (J > R) continue;
        tile_store(Atile + tri(R, J) * S::TILE_SZ, accA[s], 1.f, r16, q4, S::TILE_LD);
    }
    lds_barrier();
    {   // diagonal blocks: T_RR = (I + A_RR)^-1, lane r16 owns column r16
        const int R = wave + 4 * q4;
        if (q4 < 2 && R < NT) {
            const float* Ad = Atile + tri(R, R) * S::TILE_SZ;
            const int jc = r16;
            float t[16];
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < ii; ++m) acc += Ad[ii * S::TILE_LD + m] * t[m];
                t[ii] = (ii < jc) ? 0.f : ((ii == jc) ? 1.f : -acc);
            }
            float* Td = Ttile + tri(R, R) * S::TILE_SZ;
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) Td[ii * S::TILE_LD + jc] = t[ii];
        }
    }
    lds_barrier();
    // merge levels: blocks of m tiles, pairs (2p, 2p+1): T21 = -T22 (A21 T11)
#pragma unroll
    for (int m = 1; m < NT; m *= 2) {
        const int npair = NT / (2 * m);
        const int ntile = npair * m * m;      // output tiles per step
        // step 1: P[r][c] = sum_{x >= c} A21[r][x] T11[x][c]
        for (int t = wave; t < ntile; t += 4) {
            const int p = t / (m * m), rc = t % (m * m);
            const int r = (rc / m + rc % m) % m, c = rc % m;   // spread the long sums over waves
            const int b1 = 2 * p * m, b2 = b1 + m;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int x = c; x < m; ++x)
                tile_mma(acc, Atile + tri(b2 + r, b1 + x) * S::TILE_SZ, Ttile + tri(b1 + x, b1 + c) * S::TILE_SZ,
                         r16, q4, S::TILE_LD);
            tile_store(Pscr + (p * m * m + r * m + c) * S::TILE_SZ, acc, 1.f, r16, q4, S::TILE_LD);
        }
        lds_barrier();
        // step 2: T21[r][c] = -sum_{x <= r} T22[r][x] P[x][c]
        for (int t = wave; t < ntile; t += 4) {
            const int p = t / (m * m), rc = t % (m * m);
            const int r = rc / m, c = (rc / m + rc % m) % m;
            const int b1 = 2 * p * m, b2 = b1 + m;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int x = 0; x <= r; ++x)
                tile_mma(acc, Ttile + tri(b2 + r, b2 + x) * S::TILE_SZ, Pscr + (p * m * m + x * m + c) * S::TILE_SZ,
                         r16, q4, S::TILE_LD);
            tile_store(Ttile + tri(b2 + r, b1 + c) * S::TILE_SZ, acc, -1.f, r16, q4, S::TILE_LD);
        }
        lds_barrier();
    }

    // ------------------------------------------------------------------ phase WU
    // phase E's global stores (read back here) are visible to the whole workgroup
    __syncthreads();
    // right-hand-side fragments of phase WU (written above by this workgroup)
    uint4 bwh_f[NS][2], bwl_f[NS][2], vt_f[NS][2];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const size_t off = ch * KD * C + frag(2 * wave + ct, s, C / 32) + lane * 8;
            bwh_f[s][ct] = *reinterpret_cast<const uint4*>(ws.bwT_hi + off);
            bwl_f[s][ct] = *reinterpret_cast<const uint4*>(ws.bwT_lo + off);
            vt_f[s][ct] = *reinterpret_cast<const uint4*>(ws.vT + off);
        }

    for (int R = 0; R < NT; ++R) {
        f32x4 accw[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4 accu[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (2 * s > R) break;
            const int J = 2 * s + (q4 >> 1);
            const int jb = 32 * s + 8 * q4;
            float tv[8];
            if (J <= R) {
                const float4* tp = reinterpret_cast<const float4*>(Ttile + tri(R, J) * S::TILE_SZ + r16 * S::TILE_LD +
                                                                   8 * (q4 & 1));
                const float4 t0 = tp[0], t1 = tp[1];
                tv[0] = t0.x; tv[1] = t0.y; tv[2] = t0.z; tv[3] = t0.w;
                tv[4] = t1.x; tv[5] = t1.y; tv[6] = t1.z; tv[7] = t1.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) tv[e] = 0.f;
            }
            bf16x8 thi, tlo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                short x, y;
                split_bf(tv[e] * bet[jb + e], x, y);
                thi[e] = x;
                tlo[e] = y;
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const bf16x8 bwh = as_bf16x8(bwh_f[s][ct]), bwl = as_bf16x8(bwl_f[s][ct]);
                const bf16x8 vv = as_bf16x8(vt_f[s][ct]);
                // w^T tile (rows d, columns i) = (exp(gamma) k)^T T'^T; u tile = T' v
                accw[ct] = mfma32(bwh, thi, accw[ct]);
                accw[ct] = mfma32(bwl, thi, accw[ct]);
                accw[ct] = mfma32(bwh, tlo, accw[ct]);
                accu[ct] = mfma32(thi, vv, accu[ct]);
                accu[ct] = mfma32(tlo, vv, accu[ct]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int dt = 2 * wave + ct;   // 16-block of K (for w) and of V (for u)
            *reinterpret_cast<uint2*>(ws.w + ch * C * KD + frag(R, dt >> 1, KD / 32) + fragT(dt & 1, r16, q4)) =
                make_uint2(pack_bf2(accw[ct][0], accw[ct][1]), pack_bf2(accw[ct][2], accw[ct][3]));
            *reinterpret_cast<float4*>(ws.uT + ch * C * VD + ((size_t)(R * (VD / 16) + dt) * 64 + lane) * 4) =
                make_float4(accu[ct][0], accu[ct][1], accu[ct][2], accu[ct][3]);
        }
    }
}

template <int C, bool PER_DIM>
static hipError_t launch_intra_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                                 const float* beta, const ChunkMap& map, int nslots, int H, float scale,
                                 const Work& ws, hipStream_t stream) {
    hipLaunchKernelGGL((intra_kernel<C, PER_DIM>), dim3(nslots, H), dim3(NTHREADS), 0, stream, q, k, v, g,
                       beta, map, H, scale, ws);
    return hipGetLastError();
}

hipError_t launch_intra(int C, bool per_dim, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* g, const float* beta, const ChunkMap& map, int nslots, int H,
                        float scale, const Work& ws, hipStream_t stream) {
    if (C == 64)
        return per_dim ? launch_intra_t<64, true>(q, k, v, g, beta, map, nslots, H, scale, ws, stream)
                       : launch_intra_t<64, false>(q, k, v, g, beta, map, nslots, H, scale, ws, stream);
    return per_dim ? launch_intra_t<128, true>(q, k, v, g, beta, map, nslots, H, scale, ws, stream)
                   : launch_intra_t<128, false>(q, k, v, g, beta, map, nslots, H, scale, ws, stream);
}

}  // namespace cdr
