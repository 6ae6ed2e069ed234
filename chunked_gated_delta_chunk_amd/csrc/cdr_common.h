// Shared device helpers for the chunked gated delta-rule kernels (gfx950).
//
// MFMA operand layouts used throughout (wave64, lane l, r = l & 15, q = l >> 4):
//   v_mfma_f32_16x16x32_bf16: A[m = r][k = 8q + i], B[k = 8q + i][n = r] (i = 0..7),
//                             D[m = 4q + i][n = r] (i = 0..3)
//   v_mfma_f32_16x16x16_bf16: A[m = r][k = 4q + i], B[k = 4q + i][n = r] (i = 0..3),
//                             D as above, so a D tile is directly a K=16 B operand.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cdr {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int KD = 128;  // key dimension
constexpr int VD = 128;  // value dimension
constexpr int NTHREADS = 256;

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 with the hardware round-to-nearest-even conversion (v_cvt_pk_bf16_f32)
typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    bf16v2 r;
    r.x = (__bf16)a;
    r.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): a 16-bit-mantissa pair.
__device__ __forceinline__ void split_bf(float x, short& hi, short& lo) {
    uint16_t h = f2bf(x);
    hi = (short)h;
    lo = (short)f2bf(x - bf2f(h));
}
// the same for two values, packed two bf16 per register
__device__ __forceinline__ void split_pk(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf2(a, b);
    lo = pack_bf2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// natural exponential through the hardware base-2 exponential
__device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

__device__ __forceinline__ void unpack8(const uint4& p, float* f) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& p) {
    bf16x8 r;
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = (short)(w[i] & 0xffffu);
        r[2 * i + 1] = (short)(w[i] >> 16);
    }
    return r;
}
__device__ __forceinline__ uint4 pack8(const short* s) {
    uint4 p;
    p.x = (uint32_t)(uint16_t)s[0] | ((uint32_t)(uint16_t)s[1] << 16);
    p.y = (uint32_t)(uint16_t)s[2] | ((uint32_t)(uint16_t)s[3] << 16);
    p.z = (uint32_t)(uint16_t)s[4] | ((uint32_t)(uint16_t)s[5] << 16);
    p.w = (uint32_t)(uint16_t)s[6] | ((uint32_t)(uint16_t)s[7] << 16);
    return p;
}
__device__ __forceinline__ uint2 pack4(const short* s) {
    uint2 p;
    p.x = (uint32_t)(uint16_t)s[0] | ((uint32_t)(uint16_t)s[1] << 16);
    p.y = (uint32_t)(uint16_t)s[2] | ((uint32_t)(uint16_t)s[3] << 16);
    return p;
}

// Streaming (non-temporal) global accesses for data touched once: inputs and per-chunk
// results, so that they do not push reused data out of the caches.
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t ld_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float ld_nt(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float2 ld_nt(const float2* p) {
    const u32x2v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p));
    return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
}
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(uint2* p, const uint2& v) {
    __builtin_nontemporal_store(u32x2v{v.x, v.y}, reinterpret_cast<u32x2v*>(p));
}
__device__ __forceinline__ void st_nt(float2* p, const float2& v) {
    __builtin_nontemporal_store(u32x2v{__float_as_uint(v.x), __float_as_uint(v.y)}, reinterpret_cast<u32x2v*>(p));
}
__device__ __forceinline__ void st_nt(float4* p, const float4& v) {
    __builtin_nontemporal_store(u32x4v{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)},
                                reinterpret_cast<u32x4v*>(p));
}

// Buffer loads: the base address and size sit in a resource descriptor in scalar registers and
// each lane gives a 32-bit byte offset, so a per-lane address never takes two vector registers
// (the compiler folds a uniform base plus a lane offset of a plain global load into a 64-bit
// per-lane address, kept live per load).  A lane whose offset + access size exceeds `bytes` reads
// zero.  The third descriptor word is the raw 32-bit data format of the gfx9 family.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 bload16f(rsrc_t r, uint32_t off) {
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t off) {
    const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v.x, v.y);
}

// c + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs, accumulated in fp32
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// wait for this wave's own LDS traffic; keeps the compiler from reordering across it
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every outstanding
// global load and store of the wave, which would drain loads issued ahead of time; use this
// one wherever the threads only exchange data through LDS.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16-byte global-to-LDS copy of one 1 KiB fragment by one wave: lane l moves the 16 bytes
// at gfrag + 8 l to lfrag + 8 l (elements).  lfrag must be the same for the whole wave.  The
// copy is counted by vmcnt: wait for it with __syncthreads() (not lds_barrier()).
__device__ __forceinline__ void frag_to_lds(const uint16_t* gfrag, uint16_t* lfrag, int lane) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(gfrag + lane * 8),
                                     (__attribute__((address_space(3))) void*)(lfrag), 16, 0, 0);
}

// ---------------------------------------------------------------------------------------
// Chunk map. Tokens are packed along one axis; sequence n owns tokens [bos, bos + len).
// Fixed length: bos = n*T, len = T, and sequence n owns chunk slots
// [n*ceil(T/C), (n+1)*ceil(T/C)).  Varlen: sequence n owns the slots starting at
// floor(cu[n]/C) + n, which never overlap and stay below floor(T/C) + N.
// ---------------------------------------------------------------------------------------
struct ChunkMap {
    const int32_t* cu;  // NULL for fixed length
    int32_t T;          // tokens per sequence (fixed) or total packed tokens (varlen)
    int32_t N;          // sequences
    int32_t C;          // chunk size
    int32_t nchunk;     // ceil(T / C), fixed length only
};

// cu_seqlens entries, read at wave-uniform indices through the constant address space: they
// become scalar loads (scalar cache, waited on apart from the vector memory operations, so a
// lookup does not wait for the loads and stores a kernel keeps in flight)
__device__ __forceinline__ int cu_at(const ChunkMap& m, int i) {
    typedef const int32_t __attribute__((address_space(4))) cint32;
    return ((const cint32*)m.cu)[i];
}

__device__ __forceinline__ void seq_info(const ChunkMap& m, int n, int64_t& bos, int& len, int& slot0) {
    if (m.cu == nullptr) {
        bos = (int64_t)n * m.T;
        len = m.T;
        slot0 = n * m.nchunk;
    } else {
        const int a = cu_at(m, n), b = cu_at(m, n + 1);
        bos = a;
        len = b - a;
        slot0 = a / m.C + n;
    }
}

// Maps a chunk slot to (first token, valid rows). rows == 0 marks an unused slot.
__device__ __forceinline__ void slot_chunk(const ChunkMap& m, int slot, int64_t& tok0, int& rows) {
    int n, c;
    if (m.cu == nullptr) {
        n = slot / m.nchunk;
        c = slot - n * m.nchunk;
    } else {
        int lo = 0, hi = m.N - 1;  // largest n with cu[n]/C + n <= slot
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu_at(m, mid) / m.C + mid <= slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
        c = slot - (cu_at(m, n) / m.C + n);
    }
    int64_t bos;
    int len, slot0;
    seq_info(m, n, bos, len, slot0);
    const int start = c * m.C;
    if (c < 0 || start >= len) {
        tok0 = 0;
        rows = 0;
        return;
    }
    tok0 = bos + start;
    rows = min(m.C, len - start);
}

// ---------------------------------------------------------------------------------------
// Fragment-major storage.  Every intermediate that one kernel writes and another reads as
// an MFMA operand is stored in the order the 16x16x32 instruction consumes it: a fragment
// covers 16 non-contracted x 32 contracted indices, lane l of a wave holds non-contracted
// index l % 16 and contracted indices 8 (l / 16) .. + 7, and the 64 lane slots of 16 bytes
// follow each other.  A wave-wide load of a fragment is then one contiguous 1 KiB read.
// A matrix with the non-contracted index in 16-blocks a and the contracted index in
// 32-blocks b (nb of them) keeps fragment (a, b) at element ((a * nb + b) * 512).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ size_t frag(int a, int b, int nb) { return ((size_t)a * nb + b) * 512; }
__device__ __forceinline__ uint32_t frag32(int a, int b, int nb) { return (uint32_t)(a * nb + b) * 512u; }

// base + a 32-bit byte offset.  With a wave-uniform base the access takes the scalar-base +
// 32-bit vector-offset form, with no 64-bit address arithmetic per lane.
template <typename T>
__device__ __forceinline__ const T* cptr(const void* base, uint32_t bytes) {
    return reinterpret_cast<const T*>(static_cast<const char*>(base) + bytes);
}
template <typename T>
__device__ __forceinline__ T* mptr(void* base, uint32_t bytes) {
    return reinterpret_cast<T*>(static_cast<char*>(base) + bytes);
}
// Element offset, inside a fragment, of the four values a D-layout tile lane (r, q) holds
// when the tile is the transpose of the operand (tile rows = contracted index 16 t + 4 q + e
// within the fragment's 32, tile column = non-contracted index r): four consecutive slots.
__device__ __forceinline__ int fragT(int t, int r, int q) { return (r + 16 * (2 * t + (q >> 1))) * 8 + 4 * (q & 1); }

// Interleaved contraction order.  A 16x16 accumulator tile leaves lane (r, q) holding rows
// 4 q .. 4 q + 3 of column r, which is the operand layout of the 16x16x16 instruction.  Two
// such tiles (contracted rows 0-15 and 16-31) feed one 16x16x32 instruction directly from
// registers when the other operand lists its 32 contracted indices in the same order:
// lane slot i of lane group q holds contracted index 16 (i / 4) + 4 q + i % 4.  Arrays
// stored in this order ("pi order") are fragment-major like the others; inside fragment
// (a, b), tile t = 0, 1 of the pair puts the four values of lane (r, q) at
__device__ __forceinline__ int fragP(int t, int r, int q) { return (r + 16 * q) * 8 + 4 * t; }

// Per-chunk intermediates in the workspace; index ch = slot * H + h.  Shapes name
// (non-contracted, contracted) for fragment-major arrays.  The state update of a chunk is
// re-associated as  S' = exp(gamma_C) S - P S + B  with P = kg^T w and B = kg^T u, and its
// output as  o = Q S + U  with Q = qg - A2 w and U = A2 u, so the sequential kernel only
// needs P, B and exp(gamma_C).
struct Work {
    uint16_t* Pn;      // 2 x (K, K) frag pi bf16   -P split into high then low bf16 parts; A
                       //                       operands of -P S
    float* Bm;         // D tiles        fp32   B = kg^T u, (K/16) x (V/16) tiles of 64 lanes x 4
                       //                       rows, the layout of the state accumulator
    uint16_t* Qp;      // (C, K) frag pi bf16   Q = qg - A2 w; B operand of (Q S)^T
    uint16_t* Up;      // D tiles        bf16   U^T = (A2 u)^T, (C/16) x (V/16) tiles, the layout
                       //                       of the transposed output accumulator
    float* gC;         // [K]            fp32   exp(gamma_C)
    uint16_t* Sc;      // (V, K) frag pi bf16   state entering the chunk; A operand of (Q S)^T
    // scratch of the intra kernel (written and read back by the same workgroup)
    uint16_t* kgT;     // (K, C) frag pi bf16   exp(gamma_C - gamma) * k, high part (the low part
                       //                       stays in registers)
};

}  // namespace cdr
