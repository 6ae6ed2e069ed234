// Inter-chunk kernels, section M4 of the page "PyPTO-Gym 的 chunk_kda 算子实战".
//
// chain_kernel: the only sequential part.  One workgroup per (sequence, head, block of BV
// value columns) keeps its K x BV slice of the fp32 state in registers (value columns of
// the state evolve independently) and walks the sequence's chunks in order:
//     v_new = u - w S                      single bf16 MFMA (w, S rounded to bf16)
//     S     = exp(gamma_C) * S + kg^T v_new  split-bf16 MFMAs (hi/lo of kg^T and v_new)
// storing the chunk-entry state S (bf16) and v_new (bf16) for the output kernel.
//
// output_kernel: independent per (chunk, head, half of V):
//     o = qg S_entry + A2 v_new            bf16 MFMA, fp32 accumulate, bf16 result
#include "cdr_common.h"

namespace cdr {

template <int C, int BV>
__global__ __launch_bounds__(NTHREADS) void chain_kernel(ChunkMap map, int H, const float* __restrict__ s0,
                                                         float* __restrict__ s_out, Work ws) {
    constexpr int NVB = VD / BV;   // value blocks per head
    constexpr int VT = BV / 16;    // 16-column tiles per workgroup
    constexpr int CT = C / 64;     // 16-row tiles of the chunk per wave
    constexpr int ST_LD = KD + 8;  // padded LDS row strides (bf16)
    constexpr int VN_LD = C + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sT[BV * ST_LD];     // S^T (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t vTh[BV * VN_LD];    // v_new^T hi
    __shared__ __attribute__((aligned(16))) uint16_t vTl[BV * VN_LD];    // v_new^T lo

    const int b = blockIdx.x;
    const int vb = b % NVB, nh = b / NVB, n = nh / H, h = nh % H;
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

    for (int c = 0; c < nchunks; ++c) {
        const size_t ch = (size_t)(slot0 + c) * H + h;
        // 1. publish S (bf16) as the B operand of w S and as the chunk-entry state
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                short sb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) sb[e] = (short)f2bf(S[kt][vt][e]);
                const uint2 pk = pack4(sb);
                const int kr = 16 * (2 * wave + kt) + 4 * q4;
                const int vl = 16 * vt + r16;
                *reinterpret_cast<uint2*>(sT + vl * ST_LD + kr) = pk;
                *reinterpret_cast<uint2*>(ws.Sc + (ch * VD + v0 + vl) * KD + kr) = pk;
            }
        __syncthreads();
        // 2. v_new = u - w S
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int rt = CT * wave + ct;
            f32x4 acc[VT];
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks) {
                const int kk = 32 * ks + 8 * q4;
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(ws.w + (ch * C + 16 * rt + r16) * KD + kk));
#pragma unroll
                for (int vt = 0; vt < VT; ++vt) {
                    const bf16x8 bs = as_bf16x8(*reinterpret_cast<const uint4*>(sT + (16 * vt + r16) * ST_LD + kk));
                    acc[vt] = mfma32(a, bs, acc[vt]);
                }
            }
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                const int vl = 16 * vt + r16;
                const int cr = 16 * rt + 4 * q4;
                short hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float vn = ws.u[(ch * C + cr + e) * VD + v0 + vl] - acc[vt][e];
                    split_bf(vn, hi[e], lo[e]);
                }
                const uint2 ph = pack4(hi);
                *reinterpret_cast<uint2*>(vTh + vl * VN_LD + cr) = ph;
                *reinterpret_cast<uint2*>(vTl + vl * VN_LD + cr) = pack4(lo);
                *reinterpret_cast<uint2*>(ws.vnT + (ch * VD + v0 + vl) * C + cr) = ph;
            }
        }
        __syncthreads();
        // 3. S = exp(gamma_C) S + kg^T v_new
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int kr = 16 * (2 * wave + kt) + 4 * q4;
            const float4 gc = *reinterpret_cast<const float4*>(ws.gC + ch * KD + kr);
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                S[kt][vt][0] *= gc.x;
                S[kt][vt][1] *= gc.y;
                S[kt][vt][2] *= gc.z;
                S[kt][vt][3] *= gc.w;
            }
        }
#pragma unroll
        for (int cs = 0; cs < C / 32; ++cs) {
            const int cc = 32 * cs + 8 * q4;
            bf16x8 ah[2], al[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const size_t off = (ch * KD + 16 * (2 * wave + kt) + r16) * C + cc;
                ah[kt] = as_bf16x8(*reinterpret_cast<const uint4*>(ws.kgT_hi + off));
                al[kt] = as_bf16x8(*reinterpret_cast<const uint4*>(ws.kgT_lo + off));
            }
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                const int vl = 16 * vt + r16;
                const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4*>(vTh + vl * VN_LD + cc));
                const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4*>(vTl + vl * VN_LD + cc));
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    S[kt][vt] = mfma32(ah[kt], bh, S[kt][vt]);
                    S[kt][vt] = mfma32(al[kt], bh, S[kt][vt]);
                    S[kt][vt] = mfma32(ah[kt], bl, S[kt][vt]);
                }
            }
        }
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

template <int C>
__global__ __launch_bounds__(NTHREADS) void output_kernel(ChunkMap map, int H, uint16_t* __restrict__ o, Work ws) {
    constexpr int CT = C / 64;
    const int slot = blockIdx.x, h = blockIdx.y, vh = blockIdx.z;
    int64_t tok0;
    int rows;
    slot_chunk(map, slot, tok0, rows);
    if (rows == 0) return;
    const size_t ch = (size_t)slot * H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int vbase = 64 * vh;

    f32x4 acc[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) acc[ct][vt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // qg S_entry
#pragma unroll
    for (int ks = 0; ks < KD / 32; ++ks) {
        const int kk = 32 * ks + 8 * q4;
        bf16x8 bsv[4];
#pragma unroll
        for (int vt = 0; vt < 4; ++vt)
            bsv[vt] = as_bf16x8(*reinterpret_cast<const uint4*>(ws.Sc + (ch * VD + vbase + 16 * vt + r16) * KD + kk));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int rt = CT * wave + ct;
            const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(ws.qg + (ch * C + 16 * rt + r16) * KD + kk));
#pragma unroll
            for (int vt = 0; vt < 4; ++vt) acc[ct][vt] = mfma32(a, bsv[vt], acc[ct][vt]);
        }
    }
    // A2 v_new over the lower-triangular column blocks
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int rt = CT * wave + ct;
        for (int s = 0; s <= (rt >> 1); ++s) {
            const int J = 2 * s + (q4 >> 1);
            const int cc = 32 * s + 8 * q4;
            uint4 ar = make_uint4(0, 0, 0, 0);
            if (J <= rt) ar = *reinterpret_cast<const uint4*>(ws.A2 + (ch * C + 16 * rt + r16) * C + cc);
            const bf16x8 a = as_bf16x8(ar);
#pragma unroll
            for (int vt = 0; vt < 4; ++vt) {
                const bf16x8 bv = as_bf16x8(*reinterpret_cast<const uint4*>(ws.vnT + (ch * VD + vbase + 16 * vt + r16) * C + cc));
                acc[ct][vt] = mfma32(a, bv, acc[ct][vt]);
            }
        }
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int rt = CT * wave + ct;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int cr = 16 * rt + 4 * q4 + e;
            if (cr < rows) {
                uint16_t* orow = o + ((size_t)(tok0 + cr) * H + h) * VD + vbase;
#pragma unroll
                for (int vt = 0; vt < 4; ++vt) orow[16 * vt + r16] = f2bf(acc[ct][vt][e]);
            }
        }
    }
}

hipError_t launch_chain(int C, int BV, const ChunkMap& map, int N, int H, const float* s0, float* s_out,
                        const Work& ws, hipStream_t stream) {
    const int nvb = VD / BV;
    dim3 grid(N * H * nvb);
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
    dim3 grid(nslots, H, VD / 64);
    if (C == 64) hipLaunchKernelGGL((output_kernel<64>), grid, dim3(NTHREADS), 0, stream, map, H, o, ws);
    else hipLaunchKernelGGL((output_kernel<128>), grid, dim3(NTHREADS), 0, stream, map, H, o, ws);
    return hipGetLastError();
}

}  // namespace cdr
