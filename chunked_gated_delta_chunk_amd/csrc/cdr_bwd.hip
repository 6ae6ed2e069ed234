// Backward of the chunked gated delta rule (gradients of the per-token rule of the page
// "PyPTO-Gym 的 chunk_kda 算子实战", section 算子定位与算法背景, evaluated chunk by chunk as in
// its sections M1-M4).
//
// Per chunk (n rows, decays gamma = in-chunk prefix sum of g, kd = k e^gamma,
// kg = k e^(gamma_C - gamma), qd = scale q e^gamma, T = (I + A)^-1, W = T diag(beta) kd,
// U = T diag(beta) v, A2 the inclusive decayed q k block) the forward is the affine map
//     Delta = U - W S_in,   o = qd S_in + A2 Delta,   S_out = e^gamma_C S_in + kg^T Delta,
// i.e. S_out = (e^gamma_C - P) S_in + B with P = kg^T W, B = kg^T U, and
// o = Q S_in + A2 U with Q = qd - A2 W.  Its gradients for upstream dO and dS_out are
//     dS_in  = e^gamma_C dS_out - P^T dS_out + Q^T dO                  (reverse chain)
//     dDelta = A2^T dO + kg dS_out,  dA2 = dO Delta^T (j <= i),  dqd = dO S_in^T,
//     dkg = Delta dS_out^T,  dW = -dDelta S_in^T,  dT = dDelta (beta v)^T + dW (beta kd)^T,
//     dv = beta T^T dDelta,  dkd = beta T^T dW,  dA = -(T^T dT T^T) (j < i),
// and the decayed pair products of A (beta k_i k_j e^(gamma_i - gamma_j)) and A2 give
// the remaining k, q and gamma terms; dg is the reverse prefix sum of dgamma.
//
// Kernels (fp32 storage, products on split-bf16 MFMA: every operand is hi + lo bf16 and
// three 16x16x32 instructions give a 16-bit-mantissa product with fp32 accumulation):
//   bwd_prep   per (chunk, value head): gamma, A, A2 (pivoted pair products), T (fp32
//              diagonal blocks, the others on split-bf16 16x16x16 MFMAs), W, U, P, B and
//              Q^T dO.
//   bwd_chain  per (sequence, value head, 16 value columns): the chunk entry states S_in
//              (forward direction) and the chunk exit gradients dS_out (reverse direction),
//              fp32 states and records, -P (-P^T) with one bf16 rounding on MFMA as in the
//              forward chain; the reverse direction ends with dh0.
//   bwd_local  per (chunk, value head): all input gradients of the chunk.
//   bwd_group  sums dq, dk over the value heads of a group (grouped value heads only).
#include "chunk_dr.h"
#include "cdr_common.h"
#include "cdr_bwd_api.h"

namespace cdr {
namespace bwd {

constexpr int BWAVES = 8;
constexpr int BTHREADS = 64 * BWAVES;
constexpr int KB = 32;        // contraction block of a staged GEMM panel
constexpr int LDP = KB + 8;   // LDS pitch (bf16) of a staged panel row
constexpr int MSZ = 128 * 128;
constexpr float EPS = 1e-6f;  // in-kernel normalisation: x / sqrt(|x|^2 + eps)
// Largest gate span |gamma_i - gamma_m| over a 16-row tile and its middle row m for which the
// tile's own pairs go through the middle-row pivot: every factor is then <= e^32, so the
// decayed operands stay finite in fp32, and so do their products for the pairs that are masked.
constexpr float SAFE_SPAN = 32.f;

// per (chunk, value head) matrices, each 128 x 128 fp32 with row pitch 128
enum Mat {
    KF, QF, VF, DOF, GAM, QD, KDM, KG,                      // inputs and decayed inputs
    AH, A2M, TT, WW, UU, PP, PT, BB, BD, YY,                // prep
    SIN, DS,                                                // chains
    DL, DDL, DA2, DQD, DKG, DWM, DTM, DBT, DKT, XX,         // local
    GG, RR, CC, R2, C2, DGM, DGS,
    NMAT
};

__device__ __forceinline__ float* mat(const Work& w, size_t ch, int id) {
    return w.M + (ch * NMAT + id) * (size_t)MSZ;
}

// Operand layouts of the state chains: -P and -P^T as high bf16 parts in the first half of a
// matrix slot and low parts in the second (PP, PT), B and Q^T dO in all of it (BB, BD):
// element (m, k) of a 128 x 128 MFMA A operand stored as bf16 pi-order fragments (rows m,
// contracted index k), the layout of the forward chain's -P
__device__ __forceinline__ int pi_elem(int m, int k) {
    const int kl = k & 31;
    return (int)frag(m >> 4, k >> 5, 4) + fragP(kl >> 4, m & 15, (kl & 15) >> 2) + (kl & 3);
}
// element (m, n) of a 128 x 128 fp32 matrix stored as 16x16 accumulator tiles (the D layout:
// lane (r, q) of tile (m / 16, n / 16) holds rows 4 q .. 4 q + 3 of column r)
__device__ __forceinline__ int dtile_elem(int m, int n) {
    return ((((m >> 4) * 8 + (n >> 4)) * 64 + (n & 15) + 16 * ((m & 15) >> 2)) << 2) + (m & 3);
}

// ------------------------------------------------------------------------------------
// Split-bf16 GEMM of a workgroup: D[m][n] = sum_k A(m, k) B(n, k) (+ s2 * second pair),
// A and B read from fp32 views, staged through LDS 32 contraction indices at a time as
// hi/lo bf16, 16x16 output tiles dealt to the 8 waves.  epi(m, n, value) consumes D.
// A view must have either ks == 1 (and ms % 4 == 0) or ms == 1 (and ks % 4 == 0).  With rs set,
// row r of the matrix in memory (r = m for ks == 1, r = k for ms == 1) is read times rs[r].
struct View {
    const float* p;
    int ms, ks;
    const float* rs;
};

// A panel of M x 32 fp32 values moves global -> registers (issued early) -> LDS (split).
template <int M>
struct Panel {
    static constexpr int NF4 = M * KB / 4;
    static constexpr int PER = (NF4 + BTHREADS - 1) / BTHREADS;
    float4 x[PER];
};

template <int M>
__device__ __forceinline__ void panel_load(Panel<M>& r, const View& v, int k0, int tid) {
#pragma unroll
    for (int u = 0; u < Panel<M>::PER; ++u) {
        const int e = tid + u * BTHREADS;
        if (e < Panel<M>::NF4) {
            if (v.ks == 1) {
                const int m = e / (KB / 4), kk = (e % (KB / 4)) * 4;
                r.x[u] = *reinterpret_cast<const float4*>(v.p + (size_t)m * v.ms + k0 + kk);
                if (v.rs != nullptr) {
                    const float f = v.rs[m];
                    r.x[u] = make_float4(r.x[u].x * f, r.x[u].y * f, r.x[u].z * f, r.x[u].w * f);
                }
            } else {
                const int kk = e / (M / 4), m = (e % (M / 4)) * 4;
                r.x[u] = *reinterpret_cast<const float4*>(v.p + (size_t)(k0 + kk) * v.ks + m);
                if (v.rs != nullptr) {
                    const float f = v.rs[k0 + kk];
                    r.x[u] = make_float4(r.x[u].x * f, r.x[u].y * f, r.x[u].z * f, r.x[u].w * f);
                }
            }
        }
    }
}

template <int M>
__device__ __forceinline__ void panel_store(const Panel<M>& r, const View& v, uint16_t* hi, uint16_t* lo, int tid) {
#pragma unroll
    for (int u = 0; u < Panel<M>::PER; ++u) {
        const int e = tid + u * BTHREADS;
        if (e < Panel<M>::NF4) {
            const float4 x = r.x[u];
            if (v.ks == 1) {
                const int m = e / (KB / 4), kk = (e % (KB / 4)) * 4;
                uint32_t h0, l0, h1, l1;
                split_pk(x.x, x.y, h0, l0);
                split_pk(x.z, x.w, h1, l1);
                *reinterpret_cast<uint2*>(hi + m * LDP + kk) = make_uint2(h0, h1);
                *reinterpret_cast<uint2*>(lo + m * LDP + kk) = make_uint2(l0, l1);
            } else {
                const int kk = e / (M / 4), m = (e % (M / 4)) * 4;
                const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    short h, l;
                    split_bf(xs[q], h, l);
                    hi[(m + q) * LDP + kk] = (uint16_t)h;
                    lo[(m + q) * LDP + kk] = (uint16_t)l;
                }
            }
        }
    }
}

__device__ __forceinline__ f32x4 mfma3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl,
                                       f32x4 acc) {
    acc = mfma32(ah, bh, acc);
    acc = mfma32(al, bh, acc);
    return mfma32(ah, bl, acc);
}

// The next block's panels are loaded into registers while the current block's MFMAs run.
template <int M, int N, class Epi>
__device__ void gemm(const View a1, const View b1, int k1, const View a2, const View b2, int k2, float s2,
                     unsigned char* lds, Epi epi) {
    uint16_t* ahi = reinterpret_cast<uint16_t*>(lds);
    uint16_t* alo = ahi + M * LDP;
    uint16_t* bhi = alo + M * LDP;
    uint16_t* blo = bhi + N * LDP;
    constexpr int NTN = N / 16, NTL = (M / 16) * NTN, TPW = (NTL + BWAVES - 1) / BWAVES;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    f32x4 acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // blocks of both passes in one sequence: block q < nb1 is pass 1
    const int nb1 = k1 / KB, nb = nb1 + k2 / KB;
    Panel<M> pa;
    Panel<N> pb;
    auto issue = [&](int q) {
        if (q < nb1) {
            panel_load<M>(pa, a1, q * KB, tid);
            panel_load<N>(pb, b1, q * KB, tid);
        } else {
            panel_load<M>(pa, a2, (q - nb1) * KB, tid);
            panel_load<N>(pb, b2, (q - nb1) * KB, tid);
        }
    };
    if (nb > 0) issue(0);
    for (int q = 0; q < nb; ++q) {
        if (q == nb1 && s2 != 1.f) {  // entering the second pair: D = X1 + s2 X2 with s2 = +-1
#pragma unroll
            for (int t = 0; t < TPW; ++t) acc[t] = f32x4{acc[t][0] * s2, acc[t][1] * s2, acc[t][2] * s2, acc[t][3] * s2};
        }
        __syncthreads();
        panel_store<M>(pa, q < nb1 ? a1 : a2, ahi, alo, tid);
        panel_store<N>(pb, q < nb1 ? b1 : b2, bhi, blo, tid);
        if (q + 1 < nb) issue(q + 1);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tile = wave + BWAVES * t;
            if (tile < NTL) {
                const int I = tile / NTN, J = tile % NTN;
#pragma unroll
                for (int kk = 0; kk < KB; kk += 32) {
                    const int ro = (16 * I + (lane & 15)) * LDP + kk + 8 * (lane >> 4);
                    const int co = (16 * J + (lane & 15)) * LDP + kk + 8 * (lane >> 4);
                    acc[t] = mfma3(*reinterpret_cast<const bf16x8*>(ahi + ro), *reinterpret_cast<const bf16x8*>(alo + ro),
                                   *reinterpret_cast<const bf16x8*>(bhi + co), *reinterpret_cast<const bf16x8*>(blo + co),
                                   acc[t]);
                }
            }
        }
    }
    if (nb > nb1 && s2 != 1.f) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) acc[t] = f32x4{acc[t][0] * s2, acc[t][1] * s2, acc[t][2] * s2, acc[t][3] * s2};
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tile = wave + BWAVES * t;
        if (tile < NTL) {
            const int I = tile / NTN, J = tile % NTN;
#pragma unroll
            for (int e = 0; e < 4; ++e) epi(16 * I + 4 * (lane >> 4) + e, 16 * J + (lane & 15), acc[t][e]);
        }
    }
}

template <int M, int N, class Epi>
__device__ __forceinline__ void gemm1(const View a, const View b, int kd, unsigned char* lds, Epi epi) {
    gemm<M, N>(a, b, kd, a, b, 0, 1.f, lds, epi);
}

__device__ __forceinline__ View vw(const float* p, int ms, int ks, const float* rs = nullptr) {
    return View{p, ms, ks, rs};
}

// fp32 -> (hi, lo) bf16x8 of 8 values
__device__ __forceinline__ void split8(const float* x, bf16x8& h, bf16x8& l) {
    uint4 hh, ll;
    split_pk(x[0], x[1], hh.x, ll.x);
    split_pk(x[2], x[3], hh.y, ll.y);
    split_pk(x[4], x[5], hh.z, ll.z);
    split_pk(x[6], x[7], hh.w, ll.w);
    h = as_bf16x8(hh);
    l = as_bf16x8(ll);
}

// ------------------------------------------------------------------------------------
// Pivoted pair products.  e^(gamma_i - gamma_j) (j <= i, per key dimension) is written as
// e^(gamma_i - p) e^(p - gamma_j).  For g <= 0, gamma never increases along the chunk, so with
// i in row tile I, j in an earlier tile J < I and p the gamma of the first row of tile I (or
// of the last row of tile J), both factors are <= 1 for every gate: nothing overflows, and a
// factor that underflows belongs to a pair whose decay underflows too.  Pairs inside one
// 16-row tile have no such pivot; they are summed exactly, one exponential per pair and key
// dimension.

// ------------------------------------------------------------------------------------
template <int C, bool PER_DIM, bool L2N>
__global__ __launch_bounds__(BTHREADS) __attribute__((amdgpu_waves_per_eu(4))) void bwd_prep_kernel(In in, ChunkMap map, int H, int Hk, float scale, Work w) {
    constexpr int NT = C / 16;
    constexpr int P2 = 128 + 8;                     // pitch of pivot panels
    constexpr int INV_BYTES = C * (C + 1) * 4;   // A then T in place (pitch C + 1)
    constexpr int PIV_BYTES = 4 * 16 * P2 * 2 + 128 * 4;
    constexpr int GEMM_BYTES = 256 * LDP * 2 * 2;
    constexpr int SMEM = (INV_BYTES > PIV_BYTES ? (INV_BYTES > GEMM_BYTES ? INV_BYTES : GEMM_BYTES)
                                                : (PIV_BYTES > GEMM_BYTES ? PIV_BYTES : GEMM_BYTES));
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    __shared__ float sRq[128], sRk[128], sBeta[128], sGC[128];
    __shared__ uint32_t sWide[2];

    const int slot = blockIdx.x, hv = blockIdx.y;
    int64_t tok0;
    int rows;
    slot_chunk(map, slot, tok0, rows);
    if (rows == 0) return;
    const size_t ch = (size_t)slot * H + hv;
    const int hk = hv / (H / Hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float* gam = mat(w, ch, GAM);

    // ---- row scales and beta (a wave per row), gamma (a thread per key dimension)
    for (int i = wave; i < C; i += BWAVES) {
        float rq = 1.f, rk = 1.f, b = 0.f;
        if (i < rows) {
            const size_t tok = tok0 + i;
            if (L2N) {
                const uint16_t* qr = in.q + (tok * Hk + hk) * KD;
                const uint16_t* kr = in.k + (tok * Hk + hk) * KD;
                const float q0 = bf2f(qr[lane]), q1 = bf2f(qr[lane + 64]);
                const float k0 = bf2f(kr[lane]), k1 = bf2f(kr[lane + 64]);
                float sq = q0 * q0 + q1 * q1, sk = k0 * k0 + k1 * k1;
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) {
                    sq += __shfl_xor(sq, m, 64);
                    sk += __shfl_xor(sk, m, 64);
                }
                rq = rsqrtf(sq + EPS);
                rk = rsqrtf(sk + EPS);
            }
            b = in.beta[tok * H + hv];
        }
        if (lane == 0) {
            sRq[i] = rq;
            sRk[i] = rk;
            sBeta[i] = b;
            w.rq[ch * 128 + i] = rq;
            w.rk[ch * 128 + i] = rk;
            w.bet[ch * 128 + i] = b;
        }
    }
    if (tid < 128) {
        const int d = tid;
        float acc = 0.f;
        uint32_t wide = 0;   // tiles whose span around the middle row exceeds SAFE_SPAN
        for (int i0 = 0; i0 < C; i0 += 16) {  // one row tile: 16 independent loads in flight
            float gv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int i = i0 + u;
                const size_t tok = tok0 + min(i, rows - 1);
                const float x = PER_DIM ? in.g[(tok * H + hv) * KD + d] : in.g[tok * H + hv];
                gv[u] = (i < rows) ? x : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                acc += gv[u];
                gv[u] = acc;
                gam[(i0 + u) * 128 + d] = acc;
            }
            float span = 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) span = fmaxf(span, fabsf(gv[u] - gv[8]));
            if (!(span <= SAFE_SPAN)) wide |= 1u << (i0 >> 4);
        }
        sGC[d] = acc;
        w.gcr[ch * 128 + d] = acc;
        uint32_t wm = 0;   // the same in every lane of the wave
        for (int t = 0; t < NT; ++t)
            if (__ballot((wide >> t) & 1u) != 0) wm |= 1u << t;
        if (lane == 0) sWide[wave] = wm;
    }
    __syncthreads();
    const uint32_t wide = sWide[0] | sWide[1];
    if (tid == 0) w.wide[ch] = wide;

    // ---- inputs and their decayed forms (four elements per thread per round, loads first)
    {
        float *KFp = mat(w, ch, KF), *QFp = mat(w, ch, QF), *VFp = mat(w, ch, VF), *DOp = mat(w, ch, DOF);
        float *QDp = mat(w, ch, QD), *KDp = mat(w, ch, KDM), *KGp = mat(w, ch, KG);
        for (int e0 = tid; e0 < C * 128; e0 += 4 * BTHREADS) {
            float kf[4], qf[4], vf[4], df[4], gm[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * BTHREADS, i = e >> 7, d = e & 127;
                const size_t tok = tok0 + min(i, rows - 1);
                kf[u] = bf2f(in.k[(tok * Hk + hk) * KD + d]);
                qf[u] = bf2f(in.q[(tok * Hk + hk) * KD + d]);
                vf[u] = bf2f(in.v[(tok * H + hv) * VD + d]);
                df[u] = bf2f(in.dO[(tok * H + hv) * VD + d]);
                gm[u] = gam[e];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * BTHREADS, i = e >> 7, d = e & 127;
                const bool ok = i < rows;   // rows past the end are zero
                const float k_ = ok ? kf[u] * sRk[i] : 0.f, q_ = ok ? qf[u] * sRq[i] : 0.f;
                const float v_ = ok ? vf[u] : 0.f, d_ = ok ? df[u] : 0.f;
                const float eg = ex(gm[u]), egc = ex(sGC[d] - gm[u]);
                KFp[e] = k_;
                QFp[e] = q_;
                VFp[e] = v_;
                DOp[e] = d_;
                QDp[e] = scale * q_ * eg;
                KDp[e] = k_ * eg;
                KGp[e] = k_ * egc;
            }
        }
    }
    __syncthreads();

    // ---- A-hat (strict) and A2 (inclusive) by row tiles.  The tile rows' left factors
    // x_i e^(gamma_i - p) (shared by the waves) are staged in LDS; wave J forms its right factor
    // k_j e^(p - gamma_j) for its 16 rows in registers.  Pivot p: gamma of the tile's middle row,
    // and the diagonal tile goes through it too, unless the tile's gates are too wide (span above
    // SAFE_SPAN); then the first row (every factor <= 1) and the diagonal tile exactly.
    {
        uint16_t* kh = reinterpret_cast<uint16_t*>(smem);
        uint16_t* kl = kh + 16 * P2;
        uint16_t* qh = kl + 16 * P2;
        uint16_t* ql = qh + 16 * P2;
        float* piv = reinterpret_cast<float*>(ql + 16 * P2);
        const float* KFp = mat(w, ch, KF);
        const float* QFp = mat(w, ch, QF);
        float* AHp = mat(w, ch, AH);
        float* A2p = mat(w, ch, A2M);
        // the tiles right of the diagonal are zero (both matrices are read whole)
        for (int e = tid; e < C * C; e += BTHREADS) {
            const int i = e / C, j = e % C;
            if (j >= 16 * (i / 16 + 1)) {
                AHp[i * 128 + j] = 0.f;
                A2p[i * 128 + j] = 0.f;
            }
        }
        // the wide diagonal tiles exactly, one per wave, all at once: lane (r, q) of wave I sums
        // rows i = 16 I + 4 q + e against row j = 16 I + r; exp(-|gamma_i - gamma_j|) is the decay
        // of the later row over the earlier one (pairs with j > i are masked when stored)
        if (wave < NT && ((wide >> wave) & 1u)) {
            const int I = wave, j = 16 * I + (lane & 15);
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
            for (int d = 0; d < KD; d += 4) {
                const float4 kj = *reinterpret_cast<const float4*>(KFp + j * 128 + d);
                const float4 gj = *reinterpret_cast<const float4*>(gam + j * 128 + d);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * I + 4 * (lane >> 4) + e;
                    const float4 ki = *reinterpret_cast<const float4*>(KFp + i * 128 + d);
                    const float4 qi = *reinterpret_cast<const float4*>(QFp + i * 128 + d);
                    const float4 gi = *reinterpret_cast<const float4*>(gam + i * 128 + d);
                    const float f0 = kj.x * ex(-fabsf(gi.x - gj.x)), f1 = kj.y * ex(-fabsf(gi.y - gj.y));
                    const float f2 = kj.z * ex(-fabsf(gi.z - gj.z)), f3 = kj.w * ex(-fabsf(gi.w - gj.w));
                    ak[e] += ki.x * f0 + ki.y * f1 + ki.z * f2 + ki.w * f3;
                    aq[e] += qi.x * f0 + qi.y * f1 + qi.z * f2 + qi.w * f3;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * (lane >> 4) + e;
                AHp[i * 128 + j] = (j < i) ? ak[e] : 0.f;
                A2p[i * 128 + j] = (j <= i) ? scale * aq[e] : 0.f;
            }
        }
        // Wave J's right factors come from the same 16 rows for every row tile: their k and
        // gamma stay in registers.  The next row tile's staging inputs are loaded while the
        // current one's products run.
        constexpr int NSG = (16 * 128) / BTHREADS;   // staged elements per thread
        const int J = wave, j = 16 * J + (lane & 15);
        float kreg[KD / 32][8], greg[KD / 32][8];
        if (J < NT) {
#pragma unroll
            for (int s = 0; s < KD / 32; ++s) {
                const int d0 = 32 * s + 8 * (lane >> 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kreg[s][e] = KFp[j * 128 + d0 + e];
                    greg[s][e] = gam[j * 128 + d0 + e];
                }
            }
        }
        auto pivot_row = [&](int I) { return 16 * I + (((wide >> I) & 1u) ? 0 : 8); };
        float stk[NSG], stq[NSG], stg[NSG], stp[NSG];
        auto load_stage = [&](int I) {
#pragma unroll
            for (int u = 0; u < NSG; ++u) {
                const int e = tid + u * BTHREADS, r = e >> 7, d = e & 127, i = 16 * I + r;
                stk[u] = KFp[i * 128 + d];
                stq[u] = QFp[i * 128 + d];
                stg[u] = gam[i * 128 + d];
                stp[u] = gam[pivot_row(I) * 128 + d];
            }
        };
        const int I0 = (wide & 1u) ? 1 : 0;   // a wide first tile has no earlier one to pair with
        if (I0 < NT) load_stage(I0);
        for (int I = I0; I < NT; ++I) {
            const bool mid = !((wide >> I) & 1u);    // the same in every thread
            __syncthreads();                         // the previous tile's operands are consumed
            if (tid < 128) piv[tid] = gam[pivot_row(I) * 128 + tid];
#pragma unroll
            for (int u = 0; u < NSG; ++u) {
                const int e = tid + u * BTHREADS, r = e >> 7, d = e & 127;
                const float sc = ex(stg[u] - stp[u]);
                short h, l;
                split_bf(stk[u] * sc, h, l);
                kh[r * P2 + d] = (uint16_t)h;
                kl[r * P2 + d] = (uint16_t)l;
                split_bf(stq[u] * sc, h, l);
                qh[r * P2 + d] = (uint16_t)h;
                ql[r * P2 + d] = (uint16_t)l;
            }
            if (I + 1 < NT) load_stage(I + 1);
            __syncthreads();
            const bool run = J < I || (J == I && mid);
            if (J < NT) {
                f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
                if (run) {
#pragma unroll
                    for (int s = 0; s < KD / 32; ++s) {
                        const int d0 = 32 * s + 8 * (lane >> 4);
                        float bv[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) bv[e] = kreg[s][e] * ex(piv[d0 + e] - greg[s][e]);
                        bf16x8 b_h, b_l;
                        split8(bv, b_h, b_l);
                        const int ao = (lane & 15) * P2 + d0;
                        ak = mfma3(*reinterpret_cast<const bf16x8*>(kh + ao), *reinterpret_cast<const bf16x8*>(kl + ao),
                                   b_h, b_l, ak);
                        aq = mfma3(*reinterpret_cast<const bf16x8*>(qh + ao), *reinterpret_cast<const bf16x8*>(ql + ao),
                                   b_h, b_l, aq);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {   // the diagonal tile masked: A-hat strict, A2 inclusive
                        const int i = 16 * I + 4 * (lane >> 4) + e;
                        AHp[i * 128 + j] = (J < I || j < i) ? ak[e] : 0.f;
                        A2p[i * 128 + j] = (J < I || j <= i) ? scale * aq[e] : 0.f;
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- T = (I + A)^-1, A = beta_i A-hat (strictly lower), blocked by 16-row tiles, in place:
    // each block of T replaces the block of A it is computed from.  The diagonal blocks by
    // forward substitution in fp32 (a block's column substitution only reads rows above the one
    // it writes); then row block by row block, X_IJ = sum_{J <= K < I} A_IK T_KJ (T's unit
    // diagonal inserted) and T_IJ = -T_II X_IJ on split-bf16 16x16x16 MFMAs, wave J taking
    // tile (I, J), all X of a row block formed before any of its A blocks is overwritten.
    {
        constexpr int LP = C + 1;
        float* sT = reinterpret_cast<float*>(smem);
        const float* AHp = mat(w, ch, AH);
        for (int e = tid; e < C * C; e += BTHREADS) {
            const int i = e / C, j = e % C;
            sT[i * LP + j] = (j < i) ? sBeta[i] * AHp[i * 128 + j] : 0.f;
        }
        __syncthreads();
        if (tid < C) {
            // diagonal tile I = tid / 16 (its 16 lanes are in one wave), column c = tid % 16, row by
            // row: every lane reads row r of A before any lane overwrites it with row r of T
            const int I = tid >> 4, c = tid & 15, o = 16 * I;
#pragma unroll
            for (int r = 1; r < 16; ++r) {
                float arow[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) arow[j] = (j < r) ? sT[(o + r) * LP + o + j] : 0.f;
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (j == c) s += arow[j];                                   // A[r][c] T[c][c]
                    else if (j > c && j < r) s += arow[j] * sT[(o + j) * LP + o + c];
                }
                asm volatile("" ::: "memory");  // no load of row r may move below the stores
                if (c < r) sT[(o + r) * LP + o + c] = -s;
            }
        }
        __syncthreads();
        // lane (r16, q4): A operand row r16, columns 4 q4 .. + 3; B operand rows 4 q4 .. + 3,
        // column r16; accumulator rows 4 q4 + e, column r16
        const int r16 = lane & 15, q4 = lane >> 4;
        auto split4 = [](float a, float b, float c, float d, bf16x4& h, bf16x4& l) {
            uint2 hh, ll;
            split_pk(a, b, hh.x, ll.x);
            split_pk(c, d, hh.y, ll.y);
            h = __builtin_bit_cast(bf16x4, hh);
            l = __builtin_bit_cast(bf16x4, ll);
        };
        for (int I = 1; I < NT; ++I) {
            const int o = 16 * I, J = wave;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (J < I) {
                for (int K = J; K < I; ++K) {
                    const float* ar = sT + (o + r16) * LP + 16 * K + 4 * q4;
                    float t[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int kr = 4 * q4 + e;   // row of block T_KJ; T_JJ holds 0 on its diagonal
                        const float v = sT[(16 * K + kr) * LP + 16 * J + r16];
                        t[e] = (K == J && kr == r16) ? 1.f : v;
                    }
                    bf16x4 ah, al, bh, bl;
                    split4(ar[0], ar[1], ar[2], ar[3], ah, al);
                    split4(t[0], t[1], t[2], t[3], bh, bl);
                    x = mfma16(ah, bh, x);
                    x = mfma16(al, bh, x);
                    x = mfma16(ah, bl, x);
                }
            }
            __syncthreads();
            if (J < I) {
                float d[4];   // T_II, row r16, columns 4 q4 .. + 3 (unit lower)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 4 * q4 + e;
                    const float v = sT[(o + r16) * LP + o + c];
                    d[e] = c < r16 ? v : (c == r16 ? 1.f : 0.f);
                }
                bf16x4 ah, al, bh, bl;
                split4(d[0], d[1], d[2], d[3], ah, al);
                split4(x[0], x[1], x[2], x[3], bh, bl);   // X_IJ: its accumulator layout is the B operand's
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
                t = mfma16(ah, bh, t);
                t = mfma16(al, bh, t);
                t = mfma16(ah, bl, t);
#pragma unroll
                for (int e = 0; e < 4; ++e) sT[(o + 4 * q4 + e) * LP + 16 * J + r16] = -t[e];
            }
            __syncthreads();
        }
        float* TTp = mat(w, ch, TT);
        for (int e = tid; e < C * C; e += BTHREADS) {
            const int i = e / C, j = e % C;
            TTp[i * 128 + j] = (j < i) ? sT[i * LP + j] : (j == i ? 1.f : 0.f);
        }
    }
    __syncthreads();

    // ---- W = T (beta kd), U = T (beta v)
    {
        float* Wp = mat(w, ch, WW);
        float* Up = mat(w, ch, UU);
        const float* TTp = mat(w, ch, TT);
        const float* bet = w.bet + ch * 128;   // beta of the chunk rows: the rows of kd and v
        gemm1<C, 128>(vw(TTp, 128, 1), vw(mat(w, ch, KDM), 1, 128, bet), C, smem,
                      [&](int m, int n, float x) { Wp[m * 128 + n] = x; });
        gemm1<C, 128>(vw(TTp, 128, 1), vw(mat(w, ch, VF), 1, 128, bet), C, smem,
                      [&](int m, int n, float x) { Up[m * 128 + n] = x; });
    }
    __syncthreads();
    // ---- P = kg^T W, B = kg^T U, Y = A2^T dO.  -P and -P^T go out with one bf16 rounding as
    // the A operands of the chains (pi-order fragments), B as accumulator tiles.
    {
        uint16_t* Pp = reinterpret_cast<uint16_t*>(mat(w, ch, PP));
        uint16_t* PTp = reinterpret_cast<uint16_t*>(mat(w, ch, PT));
        float* Bp = mat(w, ch, BB);
        float* Yp = mat(w, ch, YY);
        const float* KGp = mat(w, ch, KG);
        gemm1<128, 128>(vw(KGp, 1, 128), vw(mat(w, ch, WW), 1, 128), C, smem, [&](int m, int n, float x) {
            short h, l;   // high parts in the slot's first half, low parts in its second
            split_bf(-x, h, l);
            Pp[pi_elem(m, n)] = (uint16_t)h;
            Pp[MSZ + pi_elem(m, n)] = (uint16_t)l;
            PTp[pi_elem(n, m)] = (uint16_t)h;
            PTp[MSZ + pi_elem(n, m)] = (uint16_t)l;
        });
        gemm1<128, 128>(vw(KGp, 1, 128), vw(mat(w, ch, UU), 1, 128), C, smem,
                        [&](int m, int n, float x) { Bp[dtile_elem(m, n)] = x; });
        gemm1<C, 128>(vw(mat(w, ch, A2M), 1, 128), vw(mat(w, ch, DOF), 1, 128), C, smem,
                      [&](int m, int n, float x) { Yp[m * 128 + n] = x; });
    }
    __syncthreads();
    // ---- Bd = Q^T dO = qd^T dO - W^T (A2^T dO)
    {
        float* BDp = mat(w, ch, BD);
        gemm<128, 128>(vw(mat(w, ch, QD), 1, 128), vw(mat(w, ch, DOF), 1, 128), C, vw(mat(w, ch, WW), 1, 128),
                       vw(mat(w, ch, YY), 1, 128), C, -1.f, smem,
                       [&](int m, int n, float x) { BDp[dtile_elem(m, n)] = x; });
    }
}

// ------------------------------------------------------------------------------------
// State chains, the forward chain's scheme: forward (REV = false) S <- e^gamma_C S - P S + B,
// recording the state entering every chunk; reverse dS <- e^gamma_C dS - P^T dS + Q^T dO over
// the chunks in reverse order, recording the gradient of every chunk's exit state.  One
// workgroup of 8 waves per (sequence, value head, 16 value columns); wave x keeps rows
// 16 x .. 16 x + 15 of the fp32 slice in registers (accumulator layout).  Per chunk the slice
// is recorded (fp32), published in LDS as hi + lo bf16 (the B operand of the product), and
// -P (or -P^T), stored by bwd_prep as hi + lo bf16 too, multiplies it in three MFMA chains
// (P_hi S_hi, P_lo S_hi, P_hi S_lo), as in the forward chain.  The operands of the next two chunks are in flight in a ring of three
// register buffers; the value blocks of one (sequence, head) are numbered onto one XCD.
constexpr int CH_NXCD = 8;          // workgroups are dealt to the 8 XCDs round-robin
constexpr int CH_NVB = VD / 16;     // value blocks per (sequence, head)
constexpr int CH_KS = KD / 32;      // 32-wide contraction steps over the state rows

struct ChainOps {
    uint4 ph[CH_KS];  // -P (or -P^T) fragments (x, s), high bf16 parts
    uint4 pl[CH_KS];  // and low parts
    float4 b;         // B (or Q^T dO) tile (x, value block)
    float4 gl;        // gamma_C of the wave's rows (log domain)
};

template <bool REV>
__device__ __forceinline__ void chain_load(ChainOps& op, const Work& w, size_t ch, int x, int lane, int q4, int vb) {
    const uint16_t* Pm = reinterpret_cast<const uint16_t*>(mat(w, ch, REV ? PT : PP));
#pragma unroll
    for (int s = 0; s < CH_KS; ++s) {
        op.ph[s] = *reinterpret_cast<const uint4*>(Pm + frag(x, s, CH_KS) + lane * 8);
        op.pl[s] = *reinterpret_cast<const uint4*>(Pm + MSZ + frag(x, s, CH_KS) + lane * 8);
    }
    op.b = *reinterpret_cast<const float4*>(mat(w, ch, REV ? BD : BB) + ((x * 8 + vb) * 64 + lane) * 4);
    op.gl = *reinterpret_cast<const float4*>(w.gcr + ch * 128 + 16 * x + 4 * q4);
}

template <bool REV>
__device__ __forceinline__ void chain_step(const ChainOps& op, f32x4& S, const Work& w, size_t ch, int x, int lane,
                                           int r16, int q4, int vb, uint16_t* sb) {
    // record: rows 16 x + 4 q4 + e, column 16 vb + r16 of the [k][v] matrix, past the caches
    // (bwd_local reads it after both chains; here it would only displace -P and B)
    float* rec = mat(w, ch, REV ? DS : SIN) + (16 * x + 4 * q4) * 128 + 16 * vb + r16;
#pragma unroll
    for (int e = 0; e < 4; ++e) __builtin_nontemporal_store(S[e], rec + e * 128);
    // publish: pi-order fragment x / 2 of the B operand, half x % 2
    uint2 sh, sl;
    split_pk(S[0], S[1], sh.x, sl.x);
    split_pk(S[2], S[3], sh.y, sl.y);
    const int so = (int)frag(0, x >> 1, CH_KS) + fragP(x & 1, r16, q4);
    *reinterpret_cast<uint2*>(sb + so) = sh;
    *reinterpret_cast<uint2*>(sb + CH_KS * 512 + so) = sl;
    lds_barrier();
    f32x4 a0 = {ex(op.gl.x) * S[0] + op.b.x, ex(op.gl.y) * S[1] + op.b.y, ex(op.gl.z) * S[2] + op.b.z,
                ex(op.gl.w) * S[3] + op.b.w};
    f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll
    for (int s = 0; s < CH_KS; ++s) {
        const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4*>(sb + s * 512 + lane * 8));
        const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4*>(sb + (CH_KS + s) * 512 + lane * 8));
        a0 = mfma32(as_bf16x8(op.ph[s]), bh, a0);
        a1 = mfma32(as_bf16x8(op.pl[s]), bh, a1);
        a2 = mfma32(as_bf16x8(op.ph[s]), bl, a2);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) S[e] = a0[e] + (a1[e] + a2[e]);
}

template <bool REV>
__global__ __launch_bounds__(BTHREADS) void bwd_chain_kernel(ChunkMap map, int H, const float* __restrict__ s0,
                                                              float* __restrict__ s_last, Work w) {
    __shared__ __attribute__((aligned(16))) uint16_t sbuf[2][2 * CH_KS * 512];  // two published states
    const int b = blockIdx.x;
    const int xcd = b % CH_NXCD, j = b / CH_NXCD;
    const int vb = j % CH_NVB, nh = (j / CH_NVB) * CH_NXCD + xcd;
    if (nh >= map.N * H) return;
    const int n = nh / H, hv = nh % H;
    int64_t bos;
    int len, slot0;
    seq_info(map, n, bos, len, slot0);
    const int nch = (len + map.C - 1) / map.C;
    const int tid = threadIdx.x, lane = tid & 63, x = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    // state tile: rows k = 16 x + 4 q4 + e, column v = 16 vb + r16; [N][H][V][K] in memory
    const size_t srow = (((size_t)n * H + hv) * VD + 16 * vb + r16) * KD + 16 * x + 4 * q4;
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    if (s0 != nullptr) {
        const float4 v = *reinterpret_cast<const float4*>(s0 + srow);
        S = f32x4{v.x, v.y, v.z, v.w};
    }
    // step c uses ring buffer c % 3 and publishes into LDS buffer c % 2; loads are issued
    // unconditionally (clamped to the last chunk) two steps ahead
    const int last = nch - 1;
    auto chunk_of = [&](int step) {
        const int c = max(min(step, last), 0);
        return (size_t)(slot0 + (REV ? last - c : c)) * H + hv;
    };
    ChainOps op0, op1, op2;
    auto step = [&](ChainOps& next, int cload, const ChainOps& cur, int c, int buf) {
        chain_load<REV>(next, w, chunk_of(cload), x, lane, q4, vb);
        chain_step<REV>(cur, S, w, chunk_of(c), x, lane, r16, q4, vb, sbuf[buf]);
    };
    if (nch > 0) {
        chain_load<REV>(op0, w, chunk_of(0), x, lane, q4, vb);
        chain_load<REV>(op1, w, chunk_of(1), x, lane, q4, vb);
    }
    for (int c = 0; c < nch; c += 6) {
        step(op2, c + 2, op0, c, 0);
        if (c + 1 >= nch) break;
        step(op0, c + 3, op1, c + 1, 1);
        if (c + 2 >= nch) break;
        step(op1, c + 4, op2, c + 2, 0);
        if (c + 3 >= nch) break;
        step(op2, c + 5, op0, c + 3, 1);
        if (c + 4 >= nch) break;
        step(op0, c + 6, op1, c + 4, 0);
        if (c + 5 >= nch) break;
        step(op1, c + 7, op2, c + 5, 1);
    }
    if (s_last != nullptr) *reinterpret_cast<float4*>(s_last + srow) = make_float4(S[0], S[1], S[2], S[3]);
}

// ------------------------------------------------------------------------------------
template <int C, bool PER_DIM, bool L2N>
__global__ __launch_bounds__(BTHREADS) __attribute__((amdgpu_waves_per_eu(4))) void bwd_local_kernel(In in, ChunkMap map, int H, int Hk, float scale, Work w) {
    constexpr int NT = C / 16;
    constexpr int DIAG_BYTES = NT * 256 * 2 * 4;      // diagonal blocks of G and dA2
    constexpr int SCAN_BYTES = 9 * 128 * 4;           // the dg scan's panels
    constexpr int GEMM_BYTES = 256 * LDP * 2 * 2;
    constexpr int SMEM0 = DIAG_BYTES > SCAN_BYTES ? DIAG_BYTES : SCAN_BYTES;
    constexpr int SMEM = SMEM0 > GEMM_BYTES ? SMEM0 : GEMM_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    __shared__ float sBeta[128], sGC[128];
    __shared__ float sDbA[(C / 16) * 128];   // dbeta's dA . A-hat term, [column block][row]

    const int slot = blockIdx.x, hv = blockIdx.y;
    int64_t tok0;
    int rows;
    slot_chunk(map, slot, tok0, rows);
    if (rows == 0) return;
    const size_t ch = (size_t)slot * H + hv;
    const int hk = hv / (H / Hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < 128) {
        sBeta[tid] = w.bet[ch * 128 + tid];
        sGC[tid] = w.gcr[ch * 128 + tid];
    }
    const float* gam = mat(w, ch, GAM);
    const float* SINp = mat(w, ch, SIN);
    const float* DSp = mat(w, ch, DS);

    // Delta = U - W S_in
    {
        float* DLp = mat(w, ch, DL);
        const float* Up = mat(w, ch, UU);
        gemm1<C, 128>(vw(mat(w, ch, WW), 128, 1), vw(SINp, 1, 128), KD, smem,
                      [&](int m, int n, float x) { DLp[m * 128 + n] = Up[m * 128 + n] - x; });
    }
    __syncthreads();
    // dDelta = A2^T dO + kg dS;  dA2 = dO Delta^T (j <= i);  dqd = dO S_in^T;  dkg = Delta dS^T
    {
        float* DDLp = mat(w, ch, DDL);
        float* DA2p = mat(w, ch, DA2);
        float* DQDp = mat(w, ch, DQD);
        float* DKGp = mat(w, ch, DKG);
        const float* DOp = mat(w, ch, DOF);
        const float* DLp = mat(w, ch, DL);
        gemm<C, 128>(vw(mat(w, ch, A2M), 1, 128), vw(DOp, 1, 128), C, vw(mat(w, ch, KG), 128, 1), vw(DSp, 1, 128), KD,
                     1.f, smem, [&](int m, int n, float x) { DDLp[m * 128 + n] = x; });
        gemm1<C, C>(vw(DOp, 128, 1), vw(DLp, 128, 1), VD, smem, [&](int m, int n, float x) {
            const float y = (n <= m) ? x : 0.f;
            DA2p[m * 128 + n] = y;
        });
        gemm1<C, 128>(vw(DOp, 128, 1), vw(SINp, 128, 1), VD, smem,
                      [&](int m, int n, float x) { DQDp[m * 128 + n] = x; });
        gemm1<C, 128>(vw(DLp, 128, 1), vw(DSp, 128, 1), VD, smem,
                      [&](int m, int n, float x) { DKGp[m * 128 + n] = x; });
    }
    __syncthreads();
    // dW = -dDelta S_in^T
    {
        float* DWp = mat(w, ch, DWM);
        gemm1<C, 128>(vw(mat(w, ch, DDL), 128, 1), vw(SINp, 128, 1), VD, smem,
                      [&](int m, int n, float x) { DWp[m * 128 + n] = -x; });
    }
    __syncthreads();
    // dT = dDelta (beta v)^T + dW (beta kd)^T;  T^T dDelta;  T^T dW
    {
        float* DTp = mat(w, ch, DTM);
        float* DBTp = mat(w, ch, DBT);
        float* DKTp = mat(w, ch, DKT);
        const float* TTp = mat(w, ch, TT);
        // beta_j multiplies column j of both products: applied once, to the sum
        gemm<C, C>(vw(mat(w, ch, DDL), 128, 1), vw(mat(w, ch, VF), 128, 1), VD, vw(mat(w, ch, DWM), 128, 1),
                   vw(mat(w, ch, KDM), 128, 1), KD, 1.f, smem,
                   [&](int m, int n, float x) { DTp[m * 128 + n] = sBeta[n] * x; });
        gemm1<C, 128>(vw(TTp, 1, 128), vw(mat(w, ch, DDL), 1, 128), C, smem,
                      [&](int m, int n, float x) { DBTp[m * 128 + n] = x; });
        gemm1<C, 128>(vw(TTp, 1, 128), vw(mat(w, ch, DWM), 1, 128), C, smem,
                      [&](int m, int n, float x) { DKTp[m * 128 + n] = x; });
    }
    __syncthreads();
    // X = T^T dT
    {
        float* Xp = mat(w, ch, XX);
        gemm1<C, C>(vw(mat(w, ch, TT), 1, 128), vw(mat(w, ch, DTM), 1, 128), C, smem,
                    [&](int m, int n, float x) { Xp[m * 128 + n] = x; });
    }
    __syncthreads();
    // dA = -(X T^T) (j < i);  G = beta_i dA;  and dbeta's term sum_j dA_ij A-hat_ij, per row and
    // 16-column block (the block's 16 lanes reduced; every lane of the wave takes part)
    {
        float* Gp = mat(w, ch, GG);
        const float* AHp = mat(w, ch, AH);
        gemm1<C, C>(vw(mat(w, ch, XX), 128, 1), vw(mat(w, ch, TT), 128, 1), C, smem, [&](int m, int n, float x) {
            const float da = (n < m) ? -x : 0.f;
            Gp[m * 128 + n] = sBeta[m] * da;
            float t = da * AHp[m * 128 + n];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) t += __shfl_xor(t, o, 64);
            if ((n & 15) == 0) sDbA[(n >> 4) * 128 + m] = t;
        });
    }
    __syncthreads();

    // ---- pair products with per-dimension decay
    const float* KFp = mat(w, ch, KF);
    const float* QFp = mat(w, ch, QF);
    // R_i = sum_j G_ij k_j e^(gamma_i - gamma_j), R2_i = sum_j dA2_ij k_j e^(...)   (j < i)
    // Cc_j = sum_i G_ij k_i e^(gamma_i - gamma_j), C2_j = sum_i dA2_ij q_i e^(...)  (i > j)
    // The i = j terms of R2 and C2 (no decay) are added to dq and dk in the assembly; left out
    // here they cannot cancel in dgamma, where they have no part (e^0 does not depend on gamma).
    //
    // A tile whose gates are narrow (the bit of `wide` clear, set by bwd_prep) has its own pairs
    // summed with the others below, through a pivot at its middle row.  The pairs inside a wide
    // tile are summed first, exactly: a thread per (tile, key dimension) walks the tile's 120
    // pairs, and each factor e^(gamma_i - gamma_j) is computed once for all four sums.
    const uint32_t wide = w.wide[ch];
    if (wide != 0) {
        float* sGd = reinterpret_cast<float*>(smem);   // [NT][16][16] diagonal blocks of G
        float* sDd = sGd + NT * 256;                    // and of dA2
        const float* Gp = mat(w, ch, GG);
        const float* DA2p = mat(w, ch, DA2);
        for (int e = tid; e < NT * 256; e += BTHREADS) {
            const int t = e >> 8, o = (16 * t + ((e >> 4) & 15)) * 128 + 16 * t + (e & 15);
            sGd[e] = Gp[o];
            sDd[e] = DA2p[o];
        }
        __syncthreads();
        float *Rp = mat(w, ch, RR), *R2p = mat(w, ch, R2), *Cp = mat(w, ch, CC), *C2p = mat(w, ch, C2);
        for (int it = tid; it < NT * 128; it += BTHREADS) {
            const int t = it >> 7, d = it & 127, base = 16 * t * 128 + d;
            if (!((wide >> t) & 1u)) continue;   // the same in every lane of the wave
            const float* gb = sGd + t * 256;
            const float* db = sDd + t * 256;
            float kx[16], gx[16], cc[16], c2[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                kx[r] = KFp[base + r * 128];
                gx[r] = gam[base + r * 128];
                cc[r] = 0.f;
                c2[r] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float qi = QFp[base + i * 128];
                float r1 = 0.f, r2 = 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) {
                    const float e = ex(gx[i] - gx[j]);
                    const float gij = gb[16 * i + j], dij = db[16 * i + j];
                    const float ke = kx[j] * e;
                    r1 = fmaf(gij, ke, r1);
                    r2 = fmaf(dij, ke, r2);
                    cc[j] = fmaf(gij, kx[i] * e, cc[j]);
                    c2[j] = fmaf(dij, qi * e, c2[j]);
                }
                Rp[base + i * 128] = r1;
                R2p[base + i * 128] = r2;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                Cp[base + r * 128] = cc[r];
                C2p[base + r * 128] = c2[r];
            }
        }
    }
    // Then the pairs through one pivot per tile (added to the exact part of a wide tile).  Wave w
    // owns key dimensions 16 w .. 16 w + 15 in every tile and forms its own decayed operands in
    // registers (the B fragment of a 16x16x32 MFMA: rows 8 (lane / 16) .. + 7 of a 32-row block,
    // column lane % 16); the coefficient rows (A fragments) are read straight from memory.  No
    // LDS, no barrier.  The pairs of a narrow tile with itself need no mask beyond the triangle
    // of the coefficients (G is strictly lower), except the diagonal of dA2, which is zeroed.
    __syncthreads();
    {
        const int n = lane & 15, kq = lane >> 4, d = 16 * wave + n;
        const float *Gp = mat(w, ch, GG), *DA2p = mat(w, ch, DA2);
        float *Rp = mat(w, ch, RR), *R2p = mat(w, ch, R2), *Cp = mat(w, ch, CC), *C2p = mat(w, ch, C2);
        // A fragment: row `row` of M, columns col .. col + 7, the diagonal element zeroed if asked
        auto afrag = [&](const float* M, int row, int col, bool nodiag, bf16x8& h, bf16x8& l) {
            const float4 x0 = *reinterpret_cast<const float4*>(M + row * 128 + col);
            const float4 x1 = *reinterpret_cast<const float4*>(M + row * 128 + col + 4);
            float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] = (nodiag && col + t == row) ? 0.f : x[t];
            split8(x, h, l);
        };
        // the same from the transposed matrix: column `row` of M, rows col .. col + 7 (16 lanes
        // read 16 consecutive columns of a row)
        auto afragT = [&](const float* M, int row, int col, bool nodiag, bf16x8& h, bf16x8& l) {
            float x[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] = (nodiag && col + t == row) ? 0.f : M[(col + t) * 128 + row];
            split8(x, h, l);
        };
        // rows of tile I against the rows j < lim: the earlier tiles, and the tile itself when
        // narrow; pivot: gamma of the tile's middle row when narrow, else of its first row
        for (int I = 0; I < NT; ++I) {
            const bool mid = !((wide >> I) & 1u);
            if (!mid && I == 0) continue;
            const int lim = 16 * I + (mid ? 16 : 0);
            const float p = gam[(16 * I + (mid ? 8 : 0)) * 128 + d];
            f32x4 ar = {0.f, 0.f, 0.f, 0.f}, ar2 = {0.f, 0.f, 0.f, 0.f};
            // the trip count is the same in every lane (the MFMA reads all 64)
            for (int j0 = 8 * kq; j0 < ((lim + 31) & ~31); j0 += 32) {
                float b[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int j = j0 + t;
                    const float x = KFp[j * 128 + d] * ex(p - gam[j * 128 + d]);
                    b[t] = j < lim ? x : 0.f;
                }
                bf16x8 bh, bl, ah, al;
                split8(b, bh, bl);
                afrag(Gp, 16 * I + n, j0, false, ah, al);
                ar = mfma3(ah, al, bh, bl, ar);
                afrag(DA2p, 16 * I + n, j0, true, ah, al);
                ar2 = mfma3(ah, al, bh, bl, ar2);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int o = (16 * I + 4 * kq + e) * 128 + d;
                const float f = ex(gam[o] - p);
                Rp[o] = (mid ? 0.f : Rp[o]) + f * ar[e];
                R2p[o] = (mid ? 0.f : R2p[o]) + f * ar2[e];
            }
        }
        // columns of tile J against the rows i >= lo: the later tiles, and the tile itself when
        // narrow; pivot: gamma of the tile's middle row when narrow, else of its last row
        for (int J = 0; J < NT; ++J) {
            const bool mid = !((wide >> J) & 1u);
            if (!mid && J == NT - 1) continue;
            const int lo = 16 * J + (mid ? 0 : 16);
            const float p = gam[(16 * J + (mid ? 8 : 15)) * 128 + d];
            f32x4 ac = {0.f, 0.f, 0.f, 0.f}, ac2 = {0.f, 0.f, 0.f, 0.f};
            for (int i0 = (lo & ~31) + 8 * kq; i0 < C; i0 += 32) {   // as many trips in every lane
                float bk[8], bq[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int i = i0 + t;
                    const float e = i >= lo ? ex(gam[i * 128 + d] - p) : 0.f;
                    bk[t] = KFp[i * 128 + d] * e;
                    bq[t] = QFp[i * 128 + d] * e;
                }
                bf16x8 bh, bl, ah, al;
                split8(bk, bh, bl);
                afragT(Gp, 16 * J + n, i0, false, ah, al);
                ac = mfma3(ah, al, bh, bl, ac);
                split8(bq, bh, bl);
                afragT(DA2p, 16 * J + n, i0, true, ah, al);
                ac2 = mfma3(ah, al, bh, bl, ac2);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int o = (16 * J + 4 * kq + e) * 128 + d;
                const float f = ex(p - gam[o]);
                Cp[o] = (mid ? 0.f : Cp[o]) + f * ac[e];
                C2p[o] = (mid ? 0.f : C2p[o]) + f * ac2[e];
            }
        }
    }
    __syncthreads();

    // ---- per row (a wave per row, two key dimensions per lane): the gradients of the
    // normalised q and k, the part of dgamma the scan below needs, dv, dbeta, and dq, dk (raw,
    // through the normalisation).  The gradients leave with non-temporal stores, and the matrices
    // read here for the last time come in with non-temporal loads: neither takes cache space
    // from what the kernel reads again (dkg, the scan's inputs).
    {
        const float *Rp = mat(w, ch, RR), *Cp = mat(w, ch, CC), *R2p = mat(w, ch, R2), *C2p = mat(w, ch, C2);
        const float* DA2d = mat(w, ch, DA2);
        const float *DQDp = mat(w, ch, DQD), *DKGp = mat(w, ch, DKG), *DKTp = mat(w, ch, DKT), *DBTp = mat(w, ch, DBT);
        const float* VFp = mat(w, ch, VF);
        float* DGMp = mat(w, ch, DGM);
        for (int i = wave; i < C; i += BWAVES) {
            const int r = i * 128;
            const float b = sBeta[i];
            const float a2d = DA2d[i * 129];   // dA2_ii
            float db = 0.f, dotq = 0.f, dotk = 0.f;
            float gq[2], gk[2], qv[2], kv[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int d = lane + 64 * h, e = r + d;
                const float gm = gam[e], kf = __builtin_nontemporal_load(KFp + e), qf = __builtin_nontemporal_load(QFp + e);
                const float dkt = __builtin_nontemporal_load(DKTp + e), dqd = __builtin_nontemporal_load(DQDp + e);
                const float dkg = DKGp[e];
                const float rr = __builtin_nontemporal_load(Rp + e), cc = __builtin_nontemporal_load(Cp + e);
                const float r2 = __builtin_nontemporal_load(R2p + e), c2 = __builtin_nontemporal_load(C2p + e);
                const float dbt = __builtin_nontemporal_load(DBTp + e), vf = __builtin_nontemporal_load(VFp + e);
                const float eg = ex(gm), egc = ex(sGC[d] - gm);
                // qd and kd as bwd_prep formed them (the same operations, so the same values),
                // rather than two more matrices read
                const float qd = scale * qf * eg, kd = kf * eg;
                const float dkd = b * dkt;
                gq[h] = scale * (r2 + a2d * kf) + scale * eg * dqd;
                gk[h] = rr + cc + scale * (c2 + a2d * qf) + eg * dkd + egc * dkg;
                // dgamma_i without the kg_i dkg_i term: in dg that term and its part of dgamma_C
                // sum to the prefix over earlier rows (taken in the scan below)
                DGMp[e] = kf * rr - kf * cc + scale * (qf * r2 - kf * c2) + qd * dqd + kd * dkd;
                if (i < rows) __builtin_nontemporal_store(b * dbt, in.dv + ((tok0 + i) * H + hv) * VD + d);
                db += dbt * vf + dkt * kd;
                qv[h] = qf;
                kv[h] = kf;
                dotq += qf * gq[h];
                dotk += kf * gk[h];
            }
            if (i >= rows) continue;   // the same in every lane of the wave
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                db += __shfl_xor(db, m, 64);
                if (L2N) {
                    dotq += __shfl_xor(dotq, m, 64);
                    dotk += __shfl_xor(dotk, m, 64);
                }
            }
#pragma unroll
            for (int J = 0; J < C / 16; ++J) db += sDbA[J * 128 + i];
            const size_t tok = tok0 + i;
            if (lane == 0) in.dbeta[tok * H + hv] = db;
            float* dqo = w.dqp ? w.dqp + (tok * H + hv) * KD : in.dq + (tok * Hk + hk) * KD;
            float* dko = w.dkp ? w.dkp + (tok * H + hv) * KD : in.dk + (tok * Hk + hk) * KD;
            const float rq = w.rq[ch * 128 + i], rk = w.rk[ch * 128 + i];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float xq = gq[h], xk = gk[h];
                if (L2N) {
                    xq = rq * (xq - qv[h] * dotq);
                    xk = rk * (xk - kv[h] * dotk);
                }
                __builtin_nontemporal_store(xq, dqo + lane + 64 * h);
                __builtin_nontemporal_store(xk, dko + lane + 64 * h);
            }
        }
    }
    __syncthreads();
    // ---- per key dimension: dg.  With dgamma_i' = dgamma_i + kg_i dkg_i (what the rows above
    // left in DGM) and dgamma_C = sum_i kg_i dkg_i + e^gamma_C (S_in . dS_out), the reverse prefix
    // sum
    //     dg_t = dgamma_C + sum_{i >= t} dgamma_i
    //          = e^gamma_C (S_in . dS_out) + sum_{i < t} kg_i dkg_i + sum_{i >= t} dgamma_i'
    // has no term that cancels: for strong gates every term is small where dg is, instead of the
    // difference of O(1) sums.
    {
        float (*sKg)[128] = reinterpret_cast<float (*)[128]>(smem);           // [4][128]
        float (*sSeg)[128] = reinterpret_cast<float (*)[128]>(smem) + 4;      // [4][128]
        float* sSd = reinterpret_cast<float*>(smem) + 8 * 128;
        const float *KGp = mat(w, ch, KG), *DKGp = mat(w, ch, DKG), *DGMp = mat(w, ch, DGM);
        float* DGSp = mat(w, ch, DGS);   // per-head gates: dg per row and key dimension
        // S_in . dS_out along the value columns of row d of both (a wave per row)
        for (int d = wave; d < 128; d += BWAVES) {
            float x = SINp[d * 128 + lane] * DSp[d * 128 + lane] + SINp[d * 128 + lane + 64] * DSp[d * 128 + lane + 64];
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
            if (lane == 0) sSd[d] = x;
        }
        // thread (d, part): rows part * C/4 .. + C/4 - 1, their terms held in registers
        constexpr int SEG = C / 4;
        const int d = tid & 127, part = tid >> 7, i0 = part * SEG;
        float kgd[SEG], dgm[SEG];
        float kgsum = 0.f, seg = 0.f;
#pragma unroll
        for (int u = 0; u < SEG; ++u) {
            const int i = i0 + u;
            kgd[u] = KGp[i * 128 + d] * DKGp[i * 128 + d];
            dgm[u] = (i < rows) ? DGMp[i * 128 + d] : 0.f;
            kgsum += kgd[u];
            seg += dgm[u];
        }
        sKg[part][d] = kgsum;
        sSeg[part][d] = seg;
        __syncthreads();
        float pre = 0.f;                                   // kg dkg over the rows before this part
        for (int p2 = 0; p2 < part; ++p2) pre += sKg[p2][d];
        float acc = ex(sGC[d]) * sSd[d];                   // dgamma_i' over the rows after it, and
        for (int p2 = part + 1; p2 < 4; ++p2) acc += sSeg[p2][d];   // the state-decay term
#pragma unroll
        for (int u = 0; u < SEG; ++u) {                    // exclusive prefix, rows ascending
            const float t = kgd[u];
            kgd[u] = pre;
            pre += t;
        }
#pragma unroll
        for (int u = SEG - 1; u >= 0; --u) {               // suffix, rows descending
            const int i = i0 + u;
            acc += dgm[u];
            const float dgv = acc + kgd[u];
            if (i < rows) {
                if (PER_DIM) __builtin_nontemporal_store(dgv, in.dg + ((tok0 + i) * H + hv) * KD + d);
                else DGSp[i * 128 + d] = dgv;
            }
        }
    }
    if (!PER_DIM) {
        __syncthreads();
        const float* DGSp = mat(w, ch, DGS);
        for (int i = wave; i < rows; i += BWAVES) {
            float x = DGSp[i * 128 + lane] + DGSp[i * 128 + lane + 64];
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
            if (lane == 0) in.dg[(tok0 + i) * H + hv] = x;
        }
    }
}

// dq, dk of key head hk = sum over its value heads
__global__ void bwd_group_kernel(int64_t tokens, int H, int Hk, const float* __restrict__ dqp,
                                 const float* __restrict__ dkp, float* __restrict__ dq, float* __restrict__ dk) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= tokens * Hk * KD) return;
    const int d = (int)(e % KD);
    const int64_t th = e / KD;
    const int hk = (int)(th % Hk);
    const int64_t tok = th / Hk;
    const int grp = H / Hk;
    float sq = 0.f, sk = 0.f;
    for (int gI = 0; gI < grp; ++gI) {
        const size_t o = ((size_t)tok * H + hk * grp + gI) * KD + d;
        sq += dqp[o];
        sk += dkp[o];
    }
    dq[e] = sq;
    dk[e] = sk;
}

template <int C, bool PD, bool L2>
hipError_t launch_t(const In& in, const ChunkMap& map, int nslots, int N, int H, int Hk, float scale,
                    const float* h0, const float* dht, float* dh0, const Work& w, int64_t tokens, int stages,
                    hipStream_t s) {
    // with no chunk (no token) only the reverse chain runs: dh0 = dht (or zero)
    if ((stages & 1) && nslots > 0)
        hipLaunchKernelGGL((bwd_prep_kernel<C, PD, L2>), dim3(nslots, H), dim3(BTHREADS), 0, s, in, map, H, Hk, scale,
                           w);
    if (stages & 2) {
        const int groups = (N * H + CH_NXCD - 1) / CH_NXCD;
        if (nslots > 0)
            hipLaunchKernelGGL((bwd_chain_kernel<false>), dim3(groups * CH_NXCD * CH_NVB), dim3(BTHREADS), 0, s, map, H,
                               h0, (float*)nullptr, w);
        hipLaunchKernelGGL((bwd_chain_kernel<true>), dim3(groups * CH_NXCD * CH_NVB), dim3(BTHREADS), 0, s, map, H,
                           dht, dh0, w);
    }
    if (!(stages & 4)) return hipGetLastError();
    if (nslots > 0)
        hipLaunchKernelGGL((bwd_local_kernel<C, PD, L2>), dim3(nslots, H), dim3(BTHREADS), 0, s, in, map, H, Hk, scale,
                           w);
    if (w.dqp != nullptr && tokens > 0) {
        const int64_t n = tokens * Hk * KD;
        hipLaunchKernelGGL(bwd_group_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tokens, H, Hk, w.dqp,
                           w.dkp, in.dq, in.dk);
    }
    return hipGetLastError();
}

hipError_t launch(int C, bool per_dim, bool l2n, const In& in, const ChunkMap& map, int nslots, int N, int H, int Hk,
                  float scale, const float* h0, const float* dht, float* dh0, const Work& w, int64_t tokens,
                  int stages, hipStream_t s) {
#define CDR_BWD_CASE(CC, PDV, L2V)                                                                    \
    if (C == CC && per_dim == PDV && l2n == L2V)                                                      \
        return launch_t<CC, PDV, L2V>(in, map, nslots, N, H, Hk, scale, h0, dht, dh0, w, tokens, stages, s);
    CDR_BWD_CASE(64, true, false)
    CDR_BWD_CASE(64, true, true)
    CDR_BWD_CASE(64, false, false)
    CDR_BWD_CASE(64, false, true)
    CDR_BWD_CASE(128, true, false)
    CDR_BWD_CASE(128, true, true)
    CDR_BWD_CASE(128, false, false)
    CDR_BWD_CASE(128, false, true)
#undef CDR_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace bwd

int bwd_matrices() { return bwd::NMAT; }

}  // namespace cdr
