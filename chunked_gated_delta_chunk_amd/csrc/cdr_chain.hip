// Inter-chunk kernels, section M4 of the page "PyPTO-Gym 的 chunk_kda 算子实战", with the
// chunk step re-associated (exact algebra):
//     v_new = u - w S,  S' = exp(gamma_C) S + kg^T v_new,  o = qg S + A2 v_new
//  => S' = exp(gamma_C) S - P S + B,   o = Q S + U
// with P = kg^T w, B = kg^T u, Q = qg - A2 w, U = A2 u formed by the intra kernel.
//
// chain_kernel: the only sequential part.  One workgroup of 8 waves per (sequence, head,
// block of 16 value columns); wave x keeps rows 16 x .. 16 x + 15 of the fp32 state slice in
// registers (value columns of the state evolve independently).  Per chunk:
//   1. the state is split into bf16 hi + lo and published in LDS (B operand of P S) and,
//      as bf16, to the workspace as the chunk-entry state of the output kernel;
//   2. S = exp(gamma_C) S + B - P S with three MFMA chains, P_hi S_hi, P_lo S_hi and
//      P_hi S_lo: -P and the state both keep a 16-bit mantissa as bf16 high + low parts (the
//      product of the two low parts is below fp32 rounding of the sum).
// One LDS barrier per chunk: the published state alternates between two buffers.  The
// operands of the next chunks (-P, B, exp(gamma_C)) do not depend on the state and are
// loaded two chunks ahead into a ring of three register buffers.  Workgroups are numbered
// so that all value blocks of one (sequence, head) land on the same XCD and share its L2.
//
// output_kernel: independent per (chunk, head): o^T = S_entry^T Q^T + U^T on bf16 MFMA, so
// each lane ends with four consecutive value columns of one token per value tile; pairs of
// lanes trade halves of two tiles and store 8 columns (16 bytes) each.  Q and U are read once,
// with non-temporal loads, so that they do not displace the staged state that the other
// workgroup of the same (chunk, head) finds in L2.
#include "cdr_common.h"

#include <atomic>

namespace cdr {

constexpr int NXCD = 8;     // MI355X: workgroups are dealt to the 8 XCDs round-robin
constexpr int CWAVES = 8;   // one 16-row state tile per wave
constexpr int CTHREADS = 64 * CWAVES;
constexpr int BV = 16;      // value columns per chain workgroup
constexpr int NVB = VD / BV;
constexpr int KS = KD / 32; // 32-wide contraction steps over the state rows

struct ChainOps {
    uint4 ph[KS];   // -P fragments (x, s), high bf16 parts
    uint4 pl[KS];   // and low parts
    float4 b;       // B tile (x, value block)
    float4 gc;      // exp(gamma_C) of the wave's state rows
};

// per-lane byte offsets of a wave's operands inside one chunk's arrays, the same for every chunk;
// the per-chunk bases go into buffer descriptors (scalar registers), so no 64-bit address is kept
// per lane and buffer
struct ChainOffsets {
    uint32_t p, b, g;
};

// BNT: the workgroup's slice of B, read once, comes in with a non-temporal load.  Measured: with
// more chain workgroups than the device holds at once (packed sequences), 5 % off the forward;
// with all of them resident, slower (the plain load finds B where the intra kernel left it).
template <bool MAP, bool BNT>
__device__ __forceinline__ void chain_load(ChainOps& op, const Work& ws, size_t ch, const ChainOffsets& of) {
    // one descriptor per part, so that every -P load is the lane offset plus an immediate
    const rsrc_t prh = make_rsrc(ws.Pn + ch * 2 * KD * KD, KD * KD * 2);
    const rsrc_t prl = make_rsrc(ws.Pn + ch * 2 * KD * KD + KD * KD, KD * KD * 2);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        op.ph[s] = bload16(prh, of.p + 1024u * s);
        op.pl[s] = bload16(prl, of.p + 1024u * s);
    }
    if (MAP) {
        op.b = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(ws.Bm + ch * KD * VD, KD * VD * 4), of.b, 0,
                                                                BNT ? 2 : 0);   // cache policy bit 1: non-temporal
        op.b = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
    }
    op.gc = bload16f(make_rsrc(ws.gC + ch * KD, KD * 4), of.g);
}

// sbuf: one published state, [2 (high, low)][KS fragments][512] bf16
template <bool MAP>
__device__ __forceinline__ void chain_step(const ChainOps& op, f32x4& S, const Work& ws, size_t ch, int x, int lane,
                                           int r16, int q4, int vb, uint16_t* sbuf) {
    // 1. publish the state: pi-order fragment x / 2 of the B operand, half x % 2
    uint2 sh, sl;
    split_pk(S[0], S[1], sh.x, sl.x);
    split_pk(S[2], S[3], sh.y, sl.y);
    const int so = frag(0, x >> 1, KS) + fragP(x & 1, r16, q4);
    *reinterpret_cast<uint2*>(sbuf + so) = sh;
    *reinterpret_cast<uint2*>(sbuf + KS * 512 + so) = sl;
    if (!MAP) *reinterpret_cast<uint2*>(ws.Sc + ch * VD * KD + frag(vb, x >> 1, KS) + fragP(x & 1, r16, q4)) = sh;
    lds_barrier();
    // 2. S = exp(gamma_C) S + B - P S
    f32x4 a0 = {op.gc.x * S[0] + op.b.x, op.gc.y * S[1] + op.b.y, op.gc.z * S[2] + op.b.z, op.gc.w * S[3] + op.b.w};
    f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4*>(sbuf + s * 512 + lane * 8));
        const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4*>(sbuf + (KS + s) * 512 + lane * 8));
        a0 = mfma32(as_bf16x8(op.ph[s]), bh, a0);
        a1 = mfma32(as_bf16x8(op.pl[s]), bh, a1);
        a2 = mfma32(as_bf16x8(op.ph[s]), bl, a2);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) S[e] = a0[e] + (a1[e] + a2[e]);
}

// MAP: the chunk maps without their offsets, S <- (exp(gamma_C) - P) S from S = I, which
// leaves the sequence's linear map (the final state is S_in M + X, X being the final state
// from a zero start); no chunk-entry states are written.
template <bool MAP, bool BNT>
__global__ __launch_bounds__(CTHREADS) void chain_kernel(ChunkMap map, int H, const float* __restrict__ s0,
                                                          float* __restrict__ s_out, Work ws,
                                                          const int32_t* __restrict__ order) {
    __shared__ __attribute__((aligned(16))) uint16_t sbuf[2][2 * KS * 512];  // two published states

    // workgroup b runs on XCD b % 8; the value blocks of chain nh all get the same XCD
    const int b = blockIdx.x;
    const int xcd = b % NXCD, j = b / NXCD;
    const int vb = j % NVB, nh = (j / NVB) * NXCD + xcd;
    if (nh >= map.N * H) return;
    // order (varlen): sequences by decreasing length, so the longest chains start first
    const int n = order ? order[nh / H] : nh / H, h = nh % H;
    int64_t bos;
    int len, slot0;
    seq_info(map, n, bos, len, slot0);
    const int nchunks = (len + map.C - 1) / map.C;
    const int tid = threadIdx.x, lane = tid & 63, x = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    // state tile: rows k = 16 x + 4 q4 + e, column v = 16 vb + r16; [N][H][V][K] in memory
    const size_t srow = (((size_t)n * H + h) * VD + 16 * vb + r16) * KD + 16 * x + 4 * q4;

    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    if (MAP) {
#pragma unroll
        for (int e = 0; e < 4; ++e) S[e] = (16 * x + 4 * q4 + e == 16 * vb + r16) ? 1.f : 0.f;
    } else if (s0 != nullptr) {
        const float4 v = *reinterpret_cast<const float4*>(s0 + srow);
        S = f32x4{v.x, v.y, v.z, v.w};
    }

    ChainOffsets of;
    of.p = (uint32_t)(frag(x, 0, KS) + lane * 8) * 2u;
    of.b = (uint32_t)((x * (VD / 16) + vb) * 64 + lane) * 16u;
    of.g = (uint32_t)(16 * x + 4 * q4) * 4u;
    // Chunk c is computed from ring buffer c % 3 and publishes into LDS buffer c % 2; before
    // it, chunk c + 2 is loaded into the buffer chunk c - 1 used.  Loads are issued
    // unconditionally (the index is clamped to the last chunk) so that the compiler keeps
    // them ahead of the previous chunks' work instead of sinking them next to their use.
    // (Three chunks ahead measured the same: a step's time grows with the bytes it brings into
    // the CU, not with how early they are requested.)
    ChainOps op0, op1, op2;
    const int last = nchunks - 1;
    auto chunk_of = [&](int c) { return (size_t)(slot0 + max(min(c, last), 0)) * H + h; };
    auto step = [&](ChainOps& next, int cload, const ChainOps& cur, int c, int buf) {
        chain_load<MAP, BNT>(next, ws, chunk_of(cload), of);
        chain_step<MAP>(cur, S, ws, chunk_of(c), x, lane, r16, q4, vb, sbuf[buf]);
    };
    if (nchunks > 0) {
        chain_load<MAP, BNT>(op0, ws, chunk_of(0), of);
        chain_load<MAP, BNT>(op1, ws, chunk_of(1), of);
    }
    for (int c = 0; c < nchunks; c += 6) {
        step(op2, c + 2, op0, c, 0);
        if (c + 1 >= nchunks) break;
        step(op0, c + 3, op1, c + 1, 1);
        if (c + 2 >= nchunks) break;
        step(op1, c + 4, op2, c + 2, 0);
        if (c + 3 >= nchunks) break;
        step(op2, c + 5, op0, c + 3, 1);
        if (c + 4 >= nchunks) break;
        step(op0, c + 6, op1, c + 4, 0);
        if (c + 5 >= nchunks) break;
        step(op1, c + 7, op2, c + 5, 1);
    }

    if (s_out != nullptr) *reinterpret_cast<float4*>(s_out + srow) = make_float4(S[0], S[1], S[2], S[3]);
}

// One workgroup of OWAVES waves per 64 rows of a (chunk, head): wave w takes row tile
// OWAVES part + w and all value tiles.  The chunk-entry state (A operand, shared by all
// waves) is copied into LDS in its fragment-major order; Q fragments (B operand) are read
// straight from memory and U^T initialises the accumulators.  The parts of one (chunk, head)
// are 8 workgroups apart in launch order, so they run on the same XCD and the second finds
// the staged state in that XCD's L2.  More, smaller workgroups than the CUs hold at once, so
// that some load while others store; built for five waves per SIMD (96 VGPRs, no spills:
// five workgroups per CU, the most their 32 KiB of LDS allows), one more than the
// compiler picks by itself.
constexpr int OWAVES = 4;
constexpr int OTHREADS = 64 * OWAVES;

template <int C>
__global__ __launch_bounds__(OTHREADS) __attribute__((amdgpu_waves_per_eu(5, 5))) void output_kernel(ChunkMap map, int nslots, int H, uint16_t* __restrict__ o,
                                                           Work ws) {
    constexpr int NT = C / 16;                     // row tiles of the chunk
    constexpr int NPART = NT / OWAVES;             // workgroups per (chunk, head)
    constexpr int VTW = VD / 16;                   // value tiles per wave
    constexpr int NSF = (VD / 16) * KS;            // state fragments
    static_assert(NT % OWAVES == 0, "row tiles per workgroup");
    __shared__ __attribute__((aligned(16))) uint16_t sS[NSF * 512];
    const int b = blockIdx.x, h = blockIdx.y;
    const int grp = b / (8 * NPART), r = b % (8 * NPART);
    const int part = r / 8, slot = grp * 8 + r % 8;
    if (slot >= nslots) return;
    int64_t tok0;
    int rows;
    slot_chunk(map, slot, tok0, rows);
    if (rows == 0) return;
    const size_t ch = (size_t)slot * H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int it = part * OWAVES + wave;
    for (int f = wave; f < NSF; f += OWAVES) frag_to_lds(ws.Sc + ch * VD * KD + f * 512, sS + f * 512, lane);
    uint4 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        // a Q fragment is stored half-major: the pi-order operand's two 8-byte halves of a lane
        // are 512 bytes apart
        const uint16_t* fq = ws.Qp + ch * C * KD + frag(it, s, KS);
        const u32x2v a = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(fq + lane * 4));
        const u32x2v b = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(fq + 256 + lane * 4));
        qf[s] = make_uint4(a.x, a.y, b.x, b.y);
    }
    f32x4 acc[VTW];
#pragma unroll
    for (int t = 0; t < VTW; ++t) {
        const u32x2v u = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2v*>(ws.Up + ch * C * VD + ((size_t)(it * (VD / 16) + t) * 64 + lane) * 4));
        acc[t] = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xffff0000u)};
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // direct-to-LDS copies of this wave
    __syncthreads();  // the staged state has landed
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int t = 0; t < VTW; ++t) {
            const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sS + frag(t, s, KS) + lane * 8));
            acc[t] = mfma32(a, as_bf16x8(qf[s]), acc[t]);
        }
    // acc[t]: rows v = 16 t + 4 q4 + e, column i = 16 it + r16
    // lanes q4 and q4 ^ 1 trade halves of value tiles 2p and 2p + 1, so that each lane stores 8
    // consecutive values (16 bytes): tile 2p's for even q4, tile 2p + 1's for odd q4
    const int i = 16 * it + r16;
    const bool ev = (q4 & 1) == 0;
    uint16_t* orow = o + ((size_t)(tok0 + min(i, rows - 1)) * H + h) * VD;
#pragma unroll
    for (int p = 0; p < VTW / 2; ++p) {
        const uint2 x0 = make_uint2(pack_bf2(acc[2 * p][0], acc[2 * p][1]), pack_bf2(acc[2 * p][2], acc[2 * p][3]));
        const uint2 x1 = make_uint2(pack_bf2(acc[2 * p + 1][0], acc[2 * p + 1][1]),
                                    pack_bf2(acc[2 * p + 1][2], acc[2 * p + 1][3]));
        const uint2 snd = ev ? x1 : x0;
        const uint2 rcv = make_uint2((uint32_t)__shfl_xor((int)snd.x, 16, 64), (uint32_t)__shfl_xor((int)snd.y, 16, 64));
        const uint4 val = ev ? make_uint4(x0.x, x0.y, rcv.x, rcv.y) : make_uint4(rcv.x, rcv.y, x1.x, x1.y);
        const int col = 32 * p + (ev ? 4 * q4 : 16 + 4 * (q4 - 1));
        if (i < rows) *reinterpret_cast<uint4*>(orow + col) = val;
    }
}

// Packed sequences of unequal lengths: the chain of the longest sequence bounds the kernel,
// so its workgroups should be dispatched first.  order[r] = the sequence of rank r by
// decreasing length (ties by index), from a single workgroup (N <= SEQ_ORDER_MAX).
constexpr int SEQ_ORDER_MAX = 1024;

__global__ __launch_bounds__(SEQ_ORDER_MAX) void seq_order_kernel(ChunkMap map, int32_t* __restrict__ order) {
    __shared__ int len[SEQ_ORDER_MAX];
    const int N = map.N;
    for (int n = threadIdx.x; n < N; n += SEQ_ORDER_MAX) len[n] = map.cu[n + 1] - map.cu[n];
    __syncthreads();
    for (int n = threadIdx.x; n < N; n += SEQ_ORDER_MAX) {
        const int ln = len[n];
        int r = 0;
        for (int m = 0; m < N; ++m) r += (len[m] > ln) || (len[m] == ln && m < n);
        order[r] = n;
    }
}

// the chain order for this map: NULL (sequence order) unless it is packed with N <= SEQ_ORDER_MAX
static const int32_t* chain_order(const ChunkMap& map, int N, int32_t* order_ws, hipStream_t stream) {
    if (map.cu == nullptr || order_ws == nullptr || N < 2 || N > SEQ_ORDER_MAX) return nullptr;
    hipLaunchKernelGGL(seq_order_kernel, dim3(1), dim3(SEQ_ORDER_MAX), 0, stream, map, order_ws);
    return order_ws;
}

// Chain workgroups the current device holds at once (cached per device).
static int chain_resident() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1 << 30;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int ncu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel<false, false>, CTHREADS, 0) != hipSuccess)
        return 1 << 30;
    const int r = max(1, ncu * per_cu);
    if (dev >= 0 && dev < 64) cache[dev].store(r, std::memory_order_relaxed);
    return r;
}

hipError_t launch_chain(const ChunkMap& map, int N, int H, const float* s0, float* s_out, const Work& ws,
                        int32_t* order_ws, hipStream_t stream) {
    const int groups = (N * H + NXCD - 1) / NXCD;
    const int32_t* order = chain_order(map, N, order_ws, stream);
    const int nwg = groups * NXCD * NVB;
    if (nwg > chain_resident())
        hipLaunchKernelGGL((chain_kernel<false, true>), dim3(nwg), dim3(CTHREADS), 0, stream, map, H, s0, s_out, ws, order);
    else
        hipLaunchKernelGGL((chain_kernel<false, false>), dim3(nwg), dim3(CTHREADS), 0, stream, map, H, s0, s_out, ws, order);
    return hipGetLastError();
}

hipError_t launch_chain_map(const ChunkMap& map, int N, int H, float* m_out, const Work& ws, int32_t* order_ws,
                            hipStream_t stream) {
    const int groups = (N * H + NXCD - 1) / NXCD;
    const int32_t* order = chain_order(map, N, order_ws, stream);
    hipLaunchKernelGGL((chain_kernel<true, false>), dim3(groups * NXCD * NVB), dim3(CTHREADS), 0, stream, map, H,
                       (const float*)nullptr, m_out, ws, order);
    return hipGetLastError();
}

hipError_t launch_output(int C, const ChunkMap& map, int nslots, int H, uint16_t* o, const Work& ws,
                         hipStream_t stream) {
    const int groups = (nslots + 7) / 8;  // 8 slots, then their other parts
    if (C == 64)
        hipLaunchKernelGGL((output_kernel<64>), dim3(groups * 8 * (64 / 16 / OWAVES), H), dim3(OTHREADS), 0, stream, map,
                           nslots, H, o, ws);
    else
        hipLaunchKernelGGL((output_kernel<128>), dim3(groups * 8 * (128 / 16 / OWAVES), H), dim3(OTHREADS), 0, stream,
                           map, nslots, H, o, ws);
    return hipGetLastError();
}

}  // namespace cdr
