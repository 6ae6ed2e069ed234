// Inter-chunk kernels, section M4 of the page "PyPTO-Gym 的 chunk_kda 算子实战".
//
// chain_kernel: the only sequential part.  One workgroup per (sequence, head, block of BV
// value columns) keeps its K x BV slice of the fp32 state in registers (value columns of
// the state evolve independently) and walks the sequence's chunks in order:
//     v_new = u - w S                      single bf16 MFMA (w, S rounded to bf16)
//     S     = exp(gamma_C) * S + kg^T v_new  split-bf16 MFMAs (hi/lo of kg^T and v_new)
// storing the chunk-entry state S (bf16) and v_new (bf16) for the output kernel.  The
// operands of chunk c+1 (w, kg^T, u, exp(gamma_C)) do not depend on the state, so they are
// loaded into a second register buffer while chunk c is computed.  Workgroups are numbered
// so that all value blocks of one (sequence, head) land on the same XCD and share its L2.
//
// output_kernel: independent per (chunk, head):
//     o = qg S_entry + A2 v_new            bf16 MFMA, fp32 accumulate, bf16 result
#include "cdr_common.h"

namespace cdr {

constexpr int NXCD = 8;  // MI355X: workgroups are dealt to the 8 XCDs round-robin

template <int C, int BV>
struct ChainOps {
    static constexpr int CT = C / 64;  // 16-row chunk tiles per wave
    uint4 w[CT][KD / 32];              // A operand of w S
    uint4 kh[2][C / 32];               // A operand of kg^T v_new, high part
    uint4 kl[2][C / 32];               // low part
    float4 u[CT][BV / 16];             // u^T rows (4 consecutive chunk rows)
    float4 gc[2];                      // exp(gamma_C) for the wave's state rows
};

template <int C, int BV>
__device__ __forceinline__ void chain_load(ChainOps<C, BV>& op, const Work& ws, size_t ch, int wave, int r16,
                                           int q4, int v0) {
    constexpr int CT = C / 64;
    const int lane = r16 + 16 * q4;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int rt = CT * wave + ct;
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks)
            op.w[ct][ks] = *reinterpret_cast<const uint4*>(ws.w + ch * C * KD + frag(rt, ks, KD / 32) + lane * 8);
#pragma unroll
        for (int vt = 0; vt < BV / 16; ++vt)
            op.u[ct][vt] = *reinterpret_cast<const float4*>(
                ws.uT + ch * C * VD + ((size_t)(rt * (VD / 16) + v0 / 16 + vt) * 64 + lane) * 4);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int cs = 0; cs < C / 32; ++cs) {
            const size_t off = ch * KD * C + frag(2 * wave + kt, cs, C / 32) + lane * 8;
            op.kh[kt][cs] = *reinterpret_cast<const uint4*>(ws.kgT_hi + off);
            op.kl[kt][cs] = *reinterpret_cast<const uint4*>(ws.kgT_lo + off);
        }
        op.gc[kt] = *reinterpret_cast<const float4*>(ws.gC + ch * KD + 16 * (2 * wave + kt) + 4 * q4);
    }
}

template <int C, int BV>
__device__ __forceinline__ void chain_step(const ChainOps<C, BV>& op, f32x4 (&S)[2][BV / 16], const Work& ws,
                                           size_t ch, int wave, int r16, int q4, int v0, uint16_t* sT,
                                           uint16_t* vTh, uint16_t* vTl) {
    constexpr int VT = BV / 16, CT = C / 64;
    constexpr int ST_LD = KD + 8, VN_LD = C + 8;
    // 1. publish S (bf16) as the B operand of w S and as the chunk-entry state
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            const uint2 pk = make_uint2(pack_bf2(S[kt][vt][0], S[kt][vt][1]), pack_bf2(S[kt][vt][2], S[kt][vt][3]));
            const int kr = 16 * (2 * wave + kt) + 4 * q4;
            const int vl = 16 * vt + r16;
            *reinterpret_cast<uint2*>(sT + vl * ST_LD + kr) = pk;
            // (V, K) fragment (v / 16, k / 32 = wave); this tile is its transpose
            *reinterpret_cast<uint2*>(ws.Sc + ch * VD * KD + frag(v0 / 16 + vt, wave, KD / 32) + fragT(kt, r16, q4)) = pk;
        }
    lds_barrier();
    // 2. v_new = u - w S
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int rt = CT * wave + ct;
        f32x4 acc[VT];
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks) {
            const bf16x8 a = as_bf16x8(op.w[ct][ks]);
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                const bf16x8 bs =
                    as_bf16x8(*reinterpret_cast<const uint4*>(sT + (16 * vt + r16) * ST_LD + 32 * ks + 8 * q4));
                acc[vt] = mfma32(a, bs, acc[vt]);
            }
        }
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            const int vl = 16 * vt + r16;
            const int cr = 16 * rt + 4 * q4;
            uint2 ph, pl;
            split_pk(op.u[ct][vt].x - acc[vt][0], op.u[ct][vt].y - acc[vt][1], ph.x, pl.x);
            split_pk(op.u[ct][vt].z - acc[vt][2], op.u[ct][vt].w - acc[vt][3], ph.y, pl.y);
            *reinterpret_cast<uint2*>(vTh + vl * VN_LD + cr) = ph;
            *reinterpret_cast<uint2*>(vTl + vl * VN_LD + cr) = pl;
            // (V, C) fragment (v / 16, c / 32); this tile is its transpose
            *reinterpret_cast<uint2*>(ws.vnT + ch * VD * C + frag(v0 / 16 + vt, rt >> 1, C / 32) + fragT(rt & 1, r16, q4)) = ph;
        }
    }
    lds_barrier();
    // 3. S = exp(gamma_C) S + kg^T v_new
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            S[kt][vt][0] *= op.gc[kt].x;
            S[kt][vt][1] *= op.gc[kt].y;
            S[kt][vt][2] *= op.gc[kt].z;
            S[kt][vt][3] *= op.gc[kt].w;
        }
#pragma unroll
    for (int cs = 0; cs < C / 32; ++cs) {
        const int cc = 32 * cs + 8 * q4;
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            const int vl = 16 * vt + r16;
            const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4*>(vTh + vl * VN_LD + cc));
            const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4*>(vTl + vl * VN_LD + cc));
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8 ah = as_bf16x8(op.kh[kt][cs]), al = as_bf16x8(op.kl[kt][cs]);
                S[kt][vt] = mfma32(ah, bh, S[kt][vt]);
                S[kt][vt] = mfma32(al, bh, S[kt][vt]);
                S[kt][vt] = mfma32(ah, bl, S[kt][vt]);
            }
        }
    }
}

template <int C, int BV>
__global__ __launch_bounds__(NTHREADS) void chain_kernel(ChunkMap map, int H, const float* __restrict__ s0,
                                                         float* __restrict__ s_out, Work ws) {
    constexpr int NVB = VD / BV;   // value blocks per head
    constexpr int VT = BV / 16;    // 16-column tiles per workgroup
    constexpr int ST_LD = KD + 8;  // padded LDS row strides (bf16)
    constexpr int VN_LD = C + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sT[BV * ST_LD];     // S^T (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t vTh[BV * VN_LD];    // v_new^T hi
    __shared__ __attribute__((aligned(16))) uint16_t vTl[BV * VN_LD];    // v_new^T lo

    // workgroup b runs on XCD b % 8; the value blocks of chain nh all get the same XCD
    const int b = blockIdx.x;
    const int xcd = b % NXCD, j = b / NXCD;
    const int vb = j % NVB, nh = (j / NVB) * NXCD + xcd;
    if (nh >= map.N * H) return;
    const int n = nh / H, h = nh % H;
    int64_t bos;
    int len, slot0;
    seq_info(map, n, bos, len, slot0);
    const int nchunks = (len + C - 1) / C;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int v0 = vb * BV;
    const size_t sbase = ((size_t)n * H + h) * VD;  // row of [N][H][V][K]

    f32x4 S[2][VT];  // rows k = 16 (2 wave + kt) + 4 q4 + i, column v0 + 16 vt + r16
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            const int kr = 16 * (2 * wave + kt) + 4 * q4;
            const int vc = v0 + 16 * vt + r16;
            if (s0 != nullptr) {
                const float4 x = *reinterpret_cast<const float4*>(s0 + (sbase + vc) * KD + kr);
                S[kt][vt] = f32x4{x.x, x.y, x.z, x.w};
            } else {
                S[kt][vt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }

    // Loads are issued unconditionally (the index is clamped to the last chunk) so that the
    // compiler keeps them ahead of the previous chunk's work instead of sinking them into a
    // branch next to their use.
    ChainOps<C, BV> opA, opB;
    const int last = nchunks - 1;
    auto chunk_of = [&](int c) { return (size_t)(slot0 + min(c, last)) * H + h; };
    if (nchunks > 0) chain_load<C, BV>(opA, ws, chunk_of(0), wave, r16, q4, v0);
    for (int c = 0; c < nchunks; c += 2) {
        chain_load<C, BV>(opB, ws, chunk_of(c + 1), wave, r16, q4, v0);
        chain_step<C, BV>(opA, S, ws, chunk_of(c), wave, r16, q4, v0, sT, vTh, vTl);
        if (c + 1 >= nchunks) break;
        chain_load<C, BV>(opA, ws, chunk_of(c + 2), wave, r16, q4, v0);
        chain_step<C, BV>(opB, S, ws, chunk_of(c + 1), wave, r16, q4, v0, sT, vTh, vTl);
    }

    if (s_out != nullptr) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                const int kr = 16 * (2 * wave + kt) + 4 * q4;
                const int vc = v0 + 16 * vt + r16;
                *reinterpret_cast<float4*>(s_out + (sbase + vc) * KD + kr) =
                    make_float4(S[kt][vt][0], S[kt][vt][1], S[kt][vt][2], S[kt][vt][3]);
            }
    }
}

// One workgroup per (chunk, head) computes all V columns.  The chunk-entry state and v_new
// (B operands shared by the four waves) are copied once into LDS, keeping their
// fragment-major order; qg and A2 fragments are read straight from memory.
template <int C>
__global__ __launch_bounds__(NTHREADS) void output_kernel(ChunkMap map, int H, uint16_t* __restrict__ o, Work ws) {
    constexpr int CT = C / 64;
    constexpr int SN = VD * KD, NN = VD * C;  // elements of the staged arrays
    __shared__ __attribute__((aligned(16))) uint16_t sS[SN];
    __shared__ __attribute__((aligned(16))) uint16_t sN[NN];
    const int slot = blockIdx.x, h = blockIdx.y;
    int64_t tok0;
    int rows;
    slot_chunk(map, slot, tok0, rows);
    if (rows == 0) return;
    const size_t ch = (size_t)slot * H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const uint16_t* qg = ws.qg + ch * C * KD;
    const uint16_t* a2p = ws.A2 + ch * C * C;
    {
        uint4 bs[SN / 8 / NTHREADS], bn[NN / 8 / NTHREADS];
#pragma unroll
        for (int i = 0; i < SN / 8 / NTHREADS; ++i)
            bs[i] = *reinterpret_cast<const uint4*>(ws.Sc + ch * SN + (size_t)(tid + i * NTHREADS) * 8);
#pragma unroll
        for (int i = 0; i < NN / 8 / NTHREADS; ++i)
            bn[i] = *reinterpret_cast<const uint4*>(ws.vnT + ch * NN + (size_t)(tid + i * NTHREADS) * 8);
#pragma unroll
        for (int i = 0; i < SN / 8 / NTHREADS; ++i) *reinterpret_cast<uint4*>(sS + (tid + i * NTHREADS) * 8) = bs[i];
#pragma unroll
        for (int i = 0; i < NN / 8 / NTHREADS; ++i) *reinterpret_cast<uint4*>(sN + (tid + i * NTHREADS) * 8) = bn[i];
    }
    uint4 aq[CT][KD / 32], a2[CT][C / 32];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int rt = CT * wave + ct;
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks)
            aq[ct][ks] = *reinterpret_cast<const uint4*>(qg + frag(rt, ks, KD / 32) + lane * 8);
#pragma unroll
        for (int s = 0; s < C / 32; ++s) {
            const int J = 2 * s + (q4 >> 1);
            const uint4 x = *reinterpret_cast<const uint4*>(a2p + frag(rt, s, C / 32) + lane * 8);
            a2[ct][s] = (J <= rt) ? x : make_uint4(0, 0, 0, 0);  // fragments above the diagonal are not stored
        }
    }
    lds_barrier();

    f32x4 acc[CT][VD / 16];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int vt = 0; vt < VD / 16; ++vt) acc[ct][vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KD / 32; ++ks)
#pragma unroll
        for (int vt = 0; vt < VD / 16; ++vt) {
            const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(sS + frag(vt, ks, KD / 32) + lane * 8));
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[ct][vt] = mfma32(as_bf16x8(aq[ct][ks]), b, acc[ct][vt]);
        }
#pragma unroll
    for (int s = 0; s < C / 32; ++s) {
        if (2 * s > CT * wave + CT - 1) break;
#pragma unroll
        for (int vt = 0; vt < VD / 16; ++vt) {
            const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(sN + frag(vt, s, C / 32) + lane * 8));
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[ct][vt] = mfma32(as_bf16x8(a2[ct][s]), b, acc[ct][vt]);
        }
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int rt = CT * wave + ct;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int cr = 16 * rt + 4 * q4 + e;
            if (cr < rows) {
                uint16_t* orow = o + ((size_t)(tok0 + cr) * H + h) * VD;
#pragma unroll
                for (int vt = 0; vt < VD / 16; ++vt) orow[16 * vt + r16] = f2bf(acc[ct][vt][e]);
            }
        }
    }
}

hipError_t launch_chain(int C, int BV, const ChunkMap& map, int N, int H, const float* s0, float* s_out,
                        const Work& ws, hipStream_t stream) {
    const int nvb = VD / BV;
    const int groups = (N * H + NXCD - 1) / NXCD;
    dim3 grid(groups * NXCD * nvb);
    if (C == 64) {
        if (BV == 16) hipLaunchKernelGGL((chain_kernel<64, 16>), grid, dim3(NTHREADS), 0, stream, map, H, s0, s_out, ws);
        else hipLaunchKernelGGL((chain_kernel<64, 32>), grid, dim3(NTHREADS), 0, stream, map, H, s0, s_out, ws);
    } else {
        if (BV == 16) hipLaunchKernelGGL((chain_kernel<128, 16>), grid, dim3(NTHREADS), 0, stream, map, H, s0, s_out, ws);
        else hipLaunchKernelGGL((chain_kernel<128, 32>), grid, dim3(NTHREADS), 0, stream, map, H, s0, s_out, ws);
    }
    return hipGetLastError();
}

hipError_t launch_output(int C, const ChunkMap& map, int nslots, int H, uint16_t* o, const Work& ws,
                         hipStream_t stream) {
    dim3 grid(nslots, H);
    if (C == 64) hipLaunchKernelGGL((output_kernel<64>), grid, dim3(NTHREADS), 0, stream, map, H, o, ws);
    else hipLaunchKernelGGL((output_kernel<128>), grid, dim3(NTHREADS), 0, stream, map, H, o, ws);
    return hipGetLastError();
}

}  // namespace cdr
