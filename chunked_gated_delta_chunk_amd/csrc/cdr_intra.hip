// Intra-chunk kernel: everything about one chunk of one head that does not depend on the
// state carried between chunks.  Follows sections M1-M3 of the page
// "PyPTO-Gym 的 chunk_kda 算子实战" (gate prefix sum, decayed A with its triangular
// inverse, the w / u projections) plus the chunk-local factors that section M4 consumes.
//
// One workgroup (4 waves) per (chunk slot, head).  Phases:
//   E    gate prefix sum gamma along the chunk (two halves of rows, combined through
//        LDS), per-element decay factors, and the element-wise outputs: qg, kg^T (split),
//        exp(gamma_C), (exp(gamma) k)^T (split, scratch) and v^T (scratch).
//   AA2  16x16 tiles of A (strictly lower, times beta) and A2 (lower incl. diagonal,
//        times scale) on bf16 MFMA.  Per-dimension gates enter the operands through
//        16-row pivots: for rows i in tile R and columns j in tile J <= R,
//          exp(g_i - g_j) = [exp(g_i - g_m(R)) exp(g_m(R) - g_m(J))] * exp(g_m(J) - g_j)
//        with m(.) the middle row of a tile, so no factor exceeds exp(half a tile's gate
//        span) and the product never overflows.  A uses hi/lo split operands (three
//        MFMAs); A2 feeds only the output and uses single bf16 operands.  Per-head
//        gates use raw q, k (exact bf16 products) and apply the scalar decay afterwards.
//   INV  T = (I + A)^-1: diagonal 16x16 blocks by forward substitution in fp32, then
//        T_RJ = -T_RR sum_{J<=M<R} A_RM T_MJ column block by column block on split-bf16
//        MFMAs (one column chain per wave).
//   WU   w = T diag(beta) (exp(gamma) k) and u = T diag(beta) v on split-bf16 MFMAs.
#include "cdr_common.h"

namespace cdr {

template <int C>
struct IntraShape {
    static constexpr int NT = C / 16;                  // 16-row tiles per chunk
    static constexpr int NPAIR = NT * (NT + 1) / 2;    // lower tiles incl. diagonal
    static constexpr int NOFF = NT * (NT - 1) / 2;     // strictly lower tiles
    static constexpr int HALF = C / 2;                 // rows per thread in phase E
    static constexpr int SMAX = (NPAIR + 3) / 4;       // tiles per wave in phase AA2
    static constexpr int EP_LD = KD + 4;               // padded row stride (floats)
    static constexpr int COL_LD = KD + 8;              // padded row stride (bf16)
    static constexpr int TILE_LD = 20;                 // padded 16x16 tile row stride
    static constexpr int TILE_SZ = 16 * TILE_LD;
    // LDS regions (bytes)
    static constexpr int R1 = C * EP_LD * 4;           // Ep, later A tiles
    static constexpr int R2 = 2 * C * COL_LD * 2;      // column operands, later T tiles
    static constexpr int RF = (NOFF > 0 ? NOFF : 1) * KD * 4;
    static constexpr int RG = NT * KD * 4;             // gamma at tile middles
    static constexpr int RMISC = 2 * KD * 4 + 2 * C * 4;  // half totals, gamma_C, beta, gamma rows
    static constexpr int BYTES = R1 + R2 + RF + RG + RMISC;
    static_assert(NPAIR * TILE_SZ * 4 <= R1 && NPAIR * TILE_SZ * 4 <= R2, "tile storage");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int pair_row(int p) {  // p = R(R+1)/2 + J, J <= R
    int R = 0;
    while ((R + 1) * (R + 2) / 2 <= p) ++R;
    return R;
}

template <int C, bool PER_DIM>
__global__ __launch_bounds__(NTHREADS) void intra_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, ChunkMap map, int H, float scale,
    Work ws) {
    using S = IntraShape<C>;
    constexpr int NT = S::NT, HALF = S::HALF;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::BYTES];
    float* Ep = reinterpret_cast<float*>(smem);                                   // [C][EP_LD]
    uint16_t* colh = reinterpret_cast<uint16_t*>(smem + S::R1);                   // [C][COL_LD]
    uint16_t* coll = colh + C * S::COL_LD;
    float* F = reinterpret_cast<float*>(smem + S::R1 + S::R2);                   // [NOFF][KD]
    float* gmid = reinterpret_cast<float*>(smem + S::R1 + S::R2 + S::RF);        // [NT][KD]
    float* tot = gmid + NT * KD;                                                  // [KD]
    float* glast = tot + KD;                                                      // [KD]
    float* bet = glast + KD;                                                      // [C]
    float* grow = bet + C;                                                        // [C] per-head gamma
    float* Atile = reinterpret_cast<float*>(smem);                                // after AA2
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
        const int d = tid & 127, half = tid >> 7, i0 = half * HALF;
        float gam[HALF];
        float run = 0.f;
#pragma unroll
        for (int ii = 0; ii < HALF; ++ii) {
            const int i = i0 + ii;
            float gv = 0.f;
            if (i < rows) {
                if constexpr (PER_DIM) gv = g[base + (size_t)i * rs + d];
                else gv = g[(size_t)(tok0 + i) * H + h];
            }
            run += gv;
            gam[ii] = run;
        }
        if (half == 0) tot[d] = gam[HALF - 1];
        if (tid < C) bet[tid] = (tid < rows) ? beta[(size_t)(tok0 + tid) * H + h] : 0.f;
        __syncthreads();
        if (half == 1) {
            const float t0 = tot[d];
#pragma unroll
            for (int ii = 0; ii < HALF; ++ii) gam[ii] += t0;
            glast[d] = gam[HALF - 1];
        }
#pragma unroll
        for (int tt = 0; tt < HALF / 16; ++tt) gmid[(i0 / 16 + tt) * KD + d] = gam[16 * tt + 8];
        if constexpr (!PER_DIM) {
            if (d == 0) {
#pragma unroll
                for (int ii = 0; ii < HALF; ++ii) grow[i0 + ii] = gam[ii];
            }
        }
        __syncthreads();
        const float gcl = glast[d];
        if (half == 1) ws.gC[ch * KD + d] = ex(gcl);
#pragma unroll
        for (int tt = 0; tt < HALF / 16; ++tt) {
            const float gm = gam[16 * tt + 8];
            const float e_gm = ex(gm);          // exp(gamma_m)
            const float e_cm = ex(gcl - gm);    // exp(gamma_C - gamma_m) <= 1
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                short bwh[8], bwl[8], kgh[8], kgl[8], vts[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ii = 16 * tt + 8 * hh + e;
                    const int i = i0 + ii;
                    const float x = gam[ii] - gm;
                    const float ep = ex(x);     // exp(gamma_i - gamma_m)
                    const float em = ex(-x);    // exp(gamma_m - gamma_i)
                    float kv = 0.f, qv = 0.f;
                    uint16_t vb = 0;
                    if (i < rows) {
                        kv = bf2f(k[base + (size_t)i * rs + d]);
                        qv = bf2f(q[base + (size_t)i * rs + d]);
                        vb = v[base + (size_t)i * rs + d];
                    }
                    if constexpr (PER_DIM) {
                        Ep[i * S::EP_LD + d] = ep;
                        short ch_, cl_;
                        split_bf(kv * em, ch_, cl_);
                        colh[i * S::COL_LD + d] = (uint16_t)ch_;
                        coll[i * S::COL_LD + d] = (uint16_t)cl_;
                    }
                    const float egi = e_gm * ep;                    // exp(gamma_i)
                    split_bf(kv * egi, bwh[e], bwl[e]);             // beta enters through T diag(beta)
                    ws.qg[(ch * C + i) * KD + d] = f2bf(scale * qv * egi);
                    split_bf(kv * (em * e_cm), kgh[e], kgl[e]);     // exp(gamma_C - gamma_i) k
                    vts[e] = (short)vb;
                }
                const int ib = i0 + 16 * tt + 8 * hh;
                const size_t tcol = (ch * KD + d) * C + ib;         // [ch][d][i] layouts
                *reinterpret_cast<uint4*>(ws.bwT_hi + tcol) = pack8(bwh);
                *reinterpret_cast<uint4*>(ws.bwT_lo + tcol) = pack8(bwl);
                *reinterpret_cast<uint4*>(ws.kgT_hi + tcol) = pack8(kgh);
                *reinterpret_cast<uint4*>(ws.kgT_lo + tcol) = pack8(kgl);
                *reinterpret_cast<uint4*>(ws.vT + tcol) = pack8(vts);
            }
        }
        if constexpr (PER_DIM) {
            // strictly lower pairs p = R(R-1)/2 + J, J < R: F = exp(gamma_m(R) - gamma_m(J)) <= 1
            for (int R = 1; R < NT; ++R)
                for (int J = 0; J < R; ++J) {
                    const int p = R * (R - 1) / 2 + J;
                    if ((p & 1) == half) F[p * KD + d] = ex(gmid[R * KD + d] - gmid[J * KD + d]);
                }
        }
    }
    __syncthreads();

    // ------------------------------------------------------------------ phase AA2
    f32x4 accA[S::SMAX];
#pragma unroll
    for (int s = 0; s < S::SMAX; ++s) {
        accA[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int p = wave + 4 * s;
        if (p >= S::NPAIR) continue;
        const int R = pair_row(p), J = p - R * (R + 1) / 2;
        const int i = 16 * R + r16, j = 16 * J + r16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks) {
            const int dd = 32 * ks + 8 * q4;
            uint4 kr = make_uint4(0, 0, 0, 0), qr = make_uint4(0, 0, 0, 0);
            if (i < rows) {
                kr = *reinterpret_cast<const uint4*>(k + base + (size_t)i * rs + dd);
                qr = *reinterpret_cast<const uint4*>(q + base + (size_t)i * rs + dd);
            }
            if constexpr (PER_DIM) {
                float kf[8], qf[8], ep[8], f[8];
                unpack8(kr, kf);
                unpack8(qr, qf);
                const float4* epp = reinterpret_cast<const float4*>(Ep + i * S::EP_LD + dd);
                const float4 e0 = epp[0], e1 = epp[1];
                ep[0] = e0.x; ep[1] = e0.y; ep[2] = e0.z; ep[3] = e0.w;
                ep[4] = e1.x; ep[5] = e1.y; ep[6] = e1.z; ep[7] = e1.w;
                if (J < R) {
                    const float4* fp = reinterpret_cast<const float4*>(F + (R * (R - 1) / 2 + J) * KD + dd);
                    const float4 f0 = fp[0], f1 = fp[1];
                    f[0] = f0.x; f[1] = f0.y; f[2] = f0.z; f[3] = f0.w;
                    f[4] = f1.x; f[5] = f1.y; f[6] = f1.z; f[7] = f1.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = 1.f;
                }
                bf16x8 ahi, alo, aq;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float fac = ep[e] * f[e];
                    short hh, ll;
                    split_bf(kf[e] * fac, hh, ll);
                    ahi[e] = hh;
                    alo[e] = ll;
                    aq[e] = (short)f2bf(qf[e] * fac);
                }
                const bf16x8 bhi = as_bf16x8(*reinterpret_cast<const uint4*>(colh + j * S::COL_LD + dd));
                const bf16x8 blo = as_bf16x8(*reinterpret_cast<const uint4*>(coll + j * S::COL_LD + dd));
                acc = mfma32(ahi, bhi, acc);
                acc = mfma32(alo, bhi, acc);
                acc = mfma32(ahi, blo, acc);
                acc2 = mfma32(aq, bhi, acc2);
            } else {
                uint4 kc = make_uint4(0, 0, 0, 0);
                if (j < rows) kc = *reinterpret_cast<const uint4*>(k + base + (size_t)j * rs + dd);
                const bf16x8 b = as_bf16x8(kc);
                acc = mfma32(as_bf16x8(kr), b, acc);
                acc2 = mfma32(as_bf16x8(qr), b, acc2);
            }
        }
        const int jj = 16 * J + r16;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int ii = 16 * R + 4 * q4 + rr;
            float a = acc[rr], a2 = acc2[rr];
            if constexpr (!PER_DIM) {
                const float dec = (jj <= ii) ? ex(grow[ii] - grow[jj]) : 0.f;
                a *= dec;
                a2 *= dec;
            }
            accA[s][rr] = (jj < ii) ? a * bet[ii] : 0.f;
            ws.A2[(ch * C + ii) * C + jj] = f2bf((jj <= ii) ? a2 * scale : 0.f);
        }
    }
    __syncthreads();

    // ------------------------------------------------------------------ phase INV
#pragma unroll
    for (int s = 0; s < S::SMAX; ++s) {
        const int p = wave + 4 * s;
        if (p >= S::NPAIR) continue;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) Atile[p * S::TILE_SZ + (4 * q4 + rr) * S::TILE_LD + r16] = accA[s][rr];
    }
    __syncthreads();
    {   // diagonal blocks: T_RR = (I + A_RR)^-1, lane r16 owns column r16
        const int R = wave + 4 * q4;
        if (q4 < 2 && R < NT) {
            const int pd = R * (R + 1) / 2 + R;
            const float* Ad = Atile + pd * S::TILE_SZ;
            const int jc = r16;
            float t[16];
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < ii; ++m) acc += Ad[ii * S::TILE_LD + m] * t[m];
                t[ii] = (ii < jc) ? 0.f : ((ii == jc) ? 1.f : -acc);
            }
            float* Td = Ttile + pd * S::TILE_SZ;
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) Td[ii * S::TILE_LD + jc] = t[ii];
        }
    }
    __syncthreads();
    {   // off-diagonal blocks, one column chain at a time
        // wave w owns column block w and, when there are more than four, NT - 1 - w
        for (int cj = 0; cj < 2; ++cj) {
            const int J = (cj == 0) ? wave : NT - 1 - wave;
            if (cj == 1 && J < 4) break;
            if (J >= NT) break;
            for (int R = J + 1; R < NT; ++R) {
                f32x4 P = {0.f, 0.f, 0.f, 0.f};
                for (int M = J; M < R; ++M) {
                    const float4 av = *reinterpret_cast<const float4*>(
                        Atile + (R * (R + 1) / 2 + M) * S::TILE_SZ + r16 * S::TILE_LD + 4 * q4);
                    const float* Tm = Ttile + (M * (M + 1) / 2 + J) * S::TILE_SZ;
                    const float bv[4] = {Tm[(4 * q4 + 0) * S::TILE_LD + r16], Tm[(4 * q4 + 1) * S::TILE_LD + r16],
                                         Tm[(4 * q4 + 2) * S::TILE_LD + r16], Tm[(4 * q4 + 3) * S::TILE_LD + r16]};
                    const float aa[4] = {av.x, av.y, av.z, av.w};
                    bf16x4 ah, al, bh, bl;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        short x, y;
                        split_bf(aa[e], x, y); ah[e] = x; al[e] = y;
                        split_bf(bv[e], x, y); bh[e] = x; bl[e] = y;
                    }
                    P = mfma16(ah, bh, P);
                    P = mfma16(al, bh, P);
                    P = mfma16(ah, bl, P);
                }
                const float4 tv = *reinterpret_cast<const float4*>(
                    Ttile + (R * (R + 1) / 2 + R) * S::TILE_SZ + r16 * S::TILE_LD + 4 * q4);
                const float ta[4] = {tv.x, tv.y, tv.z, tv.w};
                bf16x4 th, tl, ph, pl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    short x, y;
                    split_bf(ta[e], x, y); th[e] = x; tl[e] = y;
                    split_bf(P[e], x, y); ph[e] = x; pl[e] = y;
                }
                f32x4 X = {0.f, 0.f, 0.f, 0.f};
                X = mfma16(th, ph, X);
                X = mfma16(tl, ph, X);
                X = mfma16(th, pl, X);
                float* Tout = Ttile + (R * (R + 1) / 2 + J) * S::TILE_SZ;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Tout[(4 * q4 + rr) * S::TILE_LD + r16] = -X[rr];
                wave_lds_sync();
            }
        }
    }
    __syncthreads();

    // ------------------------------------------------------------------ phase WU
    {
        const size_t cbase = ch * KD;  // row offset of [ch][*][C] arrays in units of C
        for (int R = 0; R < NT; ++R) {
            f32x4 accw[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            f32x4 accu[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            for (int s = 0; s <= (R >> 1); ++s) {
                const int J = 2 * s + (q4 >> 1);
                const int jb = 32 * s + 8 * q4;
                float tv[8];
                if (J <= R) {
                    const float4* tp = reinterpret_cast<const float4*>(
                        Ttile + (R * (R + 1) / 2 + J) * S::TILE_SZ + r16 * S::TILE_LD + 8 * (q4 & 1));
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
                    const int d = 32 * wave + 16 * ct + r16;
                    const size_t off = (cbase + d) * C + jb;
                    const bf16x8 bwh = as_bf16x8(*reinterpret_cast<const uint4*>(ws.bwT_hi + off));
                    const bf16x8 bwl = as_bf16x8(*reinterpret_cast<const uint4*>(ws.bwT_lo + off));
                    const bf16x8 vv = as_bf16x8(*reinterpret_cast<const uint4*>(ws.vT + off));
                    accw[ct] = mfma32(thi, bwh, accw[ct]);
                    accw[ct] = mfma32(tlo, bwh, accw[ct]);
                    accw[ct] = mfma32(thi, bwl, accw[ct]);
                    accu[ct] = mfma32(thi, vv, accu[ct]);
                    accu[ct] = mfma32(tlo, vv, accu[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int d = 32 * wave + 16 * ct + r16;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int ii = 16 * R + 4 * q4 + rr;
                    ws.w[(ch * C + ii) * KD + d] = f2bf(accw[ct][rr]);
                    ws.u[(ch * C + ii) * VD + d] = accu[ct][rr];
                }
            }
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
