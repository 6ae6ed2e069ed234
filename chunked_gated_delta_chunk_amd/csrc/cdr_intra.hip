// Intra-chunk kernel: everything about one chunk of one head that does not depend on the
// state carried between chunks.  Follows sections M1-M3 of the page
// "PyPTO-Gym 的 chunk_kda 算子实战" (gate prefix sum, decayed A with its triangular
// inverse, the w / u projections) plus the chunk-local factors that section M4 consumes.
//
// One workgroup of 8 waves per (chunk slot, head); the LDS it needs leaves room for one
// workgroup per CU, so the two waves per SIMD are what hides latency.  Phases:
//   E    every thread owns a 16-row x 2-column block of the chunk (one 16-row tile); its
//        loads are issued one item ahead (g and beta when the previous item's solve starts,
//        k and v at its phase PQ).  gamma = prefix sum of g inside the tile
//        plus the totals of the tiles above (through LDS).  Per-element decay factors
//        relative to the tile's middle row m, and the element-wise outputs: exp(gamma_C),
//        kg = exp(gamma_C - gamma) k (split; fragment-major scratch read back by this
//        workgroup in INV), exp(gamma) k (single bf16: w only reaches P and Q, which are
//        formed from its own single bf16 rounding) and v, both as fragment slots kept in
//        registers until LDS is free for them after INV.
//   AA2  16x16 tiles of A (strictly lower, times beta) and A2 (lower incl. diagonal, times
//        scale) on bf16 MFMA.  Per-dimension gates enter the operands through the tile
//        pivots: for rows i in tile R and columns j in tile J <= R,
//          exp(g_i - g_j) = [exp(g_i - g_m(R)) exp(g_m(R) - g_m(J))] * exp(g_m(J) - g_j)
//        so no factor exceeds exp(half a tile's gate span) and the product never
//        overflows.  A (tile, key dimension) column whose gates span more than SAFE_SPAN
//        on a side of the middle row takes other pivots in that dimension: the gamma before
//        the tile's first row for its rows, at its last row for its columns, and its pairs
//        inside the diagonal tile are summed exactly (diag_exact).  The row operands times exp(g_i - g_m(R)) are formed once per row and
//        32-column step; a tile below the diagonal multiplies them by the pivot ratio
//        only.  A uses hi/lo split operands (three MFMAs); A2 feeds only the output
//        and uses single bf16 operands (stored transposed, scratch).  Per-head gates use
//        raw q, k (exact bf16 products) and apply the scalar decay afterwards.  Tile rows w
//        and NT-1-w form one list of NT+1 tiles shared by waves w and w+NT/2.  qg (scratch) is
//        produced on the diagonal tiles.
//   INV  the 16x16 diagonal blocks T_RR = (I + A_RR)^-1 by forward substitution in fp32
//        (wave R), then M_RJ = T_RR A_RJ (J < R) and T'_RR = T_RR diag(beta) on split-bf16
//        MFMAs, kept split in LDS.
//   WU   w = (I + A)^-1 diag(beta) exp(gamma) k and u = (I + A)^-1 diag(beta) v by blocked
//        forward substitution, Z_R = T'_RR Y_R - sum_{J<R} M_RJ Z_J, on split-bf16 MFMAs:
//        wave w owns 16 columns of each and keeps the Z tiles in registers, so the solve
//        runs without barriers.
//   PQ   the factors of the re-associated chunk step (section M4):
//          B = kg^T u                      (split-bf16: it enters the state additively)
//          P = kg^T w                      (single bf16: it is stored with one rounding)
//          Q = qg - A2 w, U = A2 u         (single bf16, they only reach the output)
//        The w and u tiles are used as MFMA operands straight from registers (pi order),
//        kg^T comes back from scratch at the start of INV and goes to LDS once the A
//        tiles there are consumed; the A2 and qg tiles stay in registers from AA2 and go to
//        LDS after the solve.  -P and B are written with ordinary stores (the chain reads
//        them next), Q and U with non-temporal ones (only the output kernel reads them).
#include "cdr_common.h"

#include <atomic>

namespace cdr {

constexpr float L2N_EPS = 1e-6f;  // in-kernel q/k normalisation: x / sqrt(|x|^2 + eps)
// Largest gate span (|gamma_i - gamma_m| over a 16-row tile and its middle row m) for which the
// tile-middle pivot factors exp(+-(gamma_i - gamma_m)) are used.  A row factor and a column factor
// are then at most e^32 each, so nothing overflows, and when the pivot ratio F between two tile
// middles underflows fp32 (below e^-87), the pair it belongs to has a true decay below
// e^(2 * 32 - 87) = e^-23, small enough to drop.  With a larger limit two moderate tiles could
// compensate a flushed F: g = -40 at rows 30 and 33 of a chunk puts 93 between the middles of
// tiles 1 and 2 while rows 30..32 stay close.  A wider (tile, key dimension) column takes pivots
// that make every factor <= 1 in that dimension, and exact sums in its diagonal tile.
constexpr float SAFE_SPAN = 32.f;
constexpr int IMAXTHREADS = 512;  // the largest workgroup (C = 128)

template <int C>
struct IntraShape {
    static constexpr int NT = C / 16;                  // 16-row tiles per chunk
    // one wave per row tile: 8 waves at C = 128; at C = 64 four, and two workgroups share a CU
    // (phases E, AA2 and INV have one row tile's work per wave either way)
    static constexpr int IW = NT;
    static constexpr int THREADS = 64 * IW;
    static constexpr int DTW = (KD / 16) / IW;          // 16-column blocks of w and u per wave
    static constexpr int NPAIR = NT * (NT + 1) / 2;    // lower tiles incl. diagonal
    static constexpr int NOFF = NT * (NT - 1) / 2;     // strictly lower tiles
    static constexpr int HF = (NT + 1) / 2;            // tiles of a row pair done by the first wave
    static constexpr int SMAX = NT + 1 - HF;           // tiles per wave in phase AA2
    // dummy stores on the item loop's entry paths (see vm_pad)
    static constexpr int NPAD = DTW * (2 * (KD / 16) + 2 * NT);
    static constexpr int EP_LD = KD + 4;               // padded row stride (floats)
    static constexpr int COL_LD = KD + 8;              // padded row stride (bf16)
    static constexpr int TILE_LD = 20;                 // padded 16x16 tile row stride
    static constexpr int TILE_SZ = 16 * TILE_LD;
    static constexpr int NS = C / 32;                  // 32-wide steps along the chunk
    // LDS regions (bytes)
    static constexpr int R1 = C * EP_LD * 4;           // Ep; later A tiles, then kg^T
    static constexpr int R2 = 2 * C * COL_LD * 2;      // column operands; later the solve, A2
    static constexpr int RF = (NOFF > NT ? NOFF : NT) * KD * 4;  // tile totals, later F
    static constexpr int RG = 2 * NT * KD * 4;         // gamma and exp(gamma) at tile middles
    static constexpr int RMISC = 3 * C * 4;            // beta, per-head gamma, key row scales
    static constexpr int BYTES = R1 + R2 + RF + RG + RMISC;
    // phase INV/WU in R2: T_RR (fp32 tiles), then -M_RJ (J < R) and T'_RR split into bf16
    // high and low parts, 1 KiB per tile
    static constexpr int TD_BYTES = NT * TILE_SZ * 4;
    static constexpr int SOLVE_BYTES = TD_BYTES + (NOFF + NT) * 1024;
    static_assert(NPAIR * TILE_SZ * 4 <= R1, "A tiles");
    static_assert(SOLVE_BYTES <= R2, "solve operands");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int tri(int R, int J) { return R * (R + 1) / 2 + J; }  // J <= R

// x = hi + lo as split_pk, with the two high parts converted by one packed conversion whose
// halves give them back as floats.  The packed value passes through an empty asm statement
// (no instruction is emitted) so that the compiler does not convert each value on its own
// (two conversions, two shifts and a permute per pair instead of one, one, one).  The
// conversion itself stays compiler-generated: an instruction inside inline asm is outside the
// compiler's hazard checks, and reading an MFMA result that way returns stale values.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    uint32_t h = pack_bf2(a, b);
    asm("" : "+v"(h));
    hi = h;
    lo = pack_bf2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
}

__device__ __forceinline__ void tile_store(float* Tt, const f32x4& v, float sgn, int r16, int q4, int ld) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) Tt[(4 * q4 + rr) * ld + r16] = sgn * v[rr];
}

// qg values of lane (r, q) of a diagonal tile R, columns 32 ks + 8 q .. + 7, into the
// accumulator layout of (qg)^T tiles (rows d, columns i): tile (R, d / 16), lane
// (i % 16) + 16 ((d % 16) / 4), element d % 4
__device__ __forceinline__ void store_qg(uint16_t* base, int R, int ks, int r, int q, const uint4& pq) {
    uint16_t* t = base + (size_t)(R * (KD / 16) + 2 * ks + (q >> 1)) * 256;
    *reinterpret_cast<uint2*>(t + (r + 16 * (2 * (q & 1))) * 4) = make_uint2(pq.x, pq.y);
    *reinterpret_cast<uint2*>(t + (r + 16 * (2 * (q & 1) + 1)) * 4) = make_uint2(pq.z, pq.w);
}

// Position of A2 fragment (I, s), s <= I / 2, in the list of lower fragments
__device__ __forceinline__ int a2_slot(int I, int s) {
    const int h = I >> 1;
    return I + ((I & 1) ? h * h : h * (h - 1)) + s;
}

__device__ __forceinline__ uint4 neg_bf16x8(const uint4& a) {
    return make_uint4(a.x ^ 0x80008000u, a.y ^ 0x80008000u, a.z ^ 0x80008000u, a.w ^ 0x80008000u);
}

// Phase E inputs of one item, held in registers: thread (R = wave, d0 = 2 (lane)) owns rows
// 16 R .. 16 R + 15 and columns d0, d0 + 1; loaded one item ahead, the gates and beta early
// (when the solve starts) and k and v later (at phase PQ), so that each workgroup's loads
// reach memory in two smaller bursts and ahead of its result stores.  Rows past the end of the sequence read its last row (masked
// when used), so the loads stay unconditional.
struct EIn {
    float2 g[16];
    uint32_t k[16], v[16];
    float b;
};

// Where an item's rows are.  Every item exists when this is called with item >= 0; no item
// (-1) reads token 0 of item 0, which exists whenever there are items, so that the loads
// stay unconditional and every register of EIn is written on every path.
struct ELoc {
    int64_t tok0;
    int rows, h;
};

__device__ __forceinline__ ELoc e_locate(const ChunkMap& map, int H, int item) {
    item = max(item, 0);
    ELoc l;
    l.h = item % H;
    slot_chunk(map, item / H, l.tok0, l.rows);
    return l;
}

template <int C, bool PER_DIM>
__device__ __forceinline__ void e_load_g(EIn& in, const float* g, const float* beta, const ELoc& l, int H, int tid) {
    // per lane only 32-bit byte offsets of rows min(16 R + ii, last) from uniform item bases
    const uint32_t last = (uint32_t)max(l.rows - 1, 0);
    const uint32_t rs = (uint32_t)H * KD;
    const uint32_t R = (uint32_t)min(tid >> 6, C / 16 - 1), d0 = 2u * (uint32_t)(tid & 63);
    in.b = *cptr<float>(beta + ((size_t)l.tok0 * H + l.h), min((uint32_t)tid, last) * (uint32_t)H * 4u);
    const uint32_t r0 = 16u * R;
    const uint32_t og0 = (r0 * rs + d0) * 4u, ogl = (last * rs + d0) * 4u;   // g bytes (per dimension)
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
        if constexpr (PER_DIM) {
            // the gates (the largest input, read once) past the caches: they leave the
            // memory-side cache to -P and B, which the chain reads next
            in.g[ii] = ld_nt(cptr<float2>(g + ((size_t)l.tok0 * rs + (size_t)l.h * KD), min(og0 + ii * rs * 4u, ogl)));
        } else {
            const float s1 = *cptr<float>(g + ((size_t)l.tok0 * H + l.h), min(r0 + ii, last) * (uint32_t)H * 4u);
            in.g[ii] = make_float2(s1, s1);
        }
    }
}

template <int C>
__device__ __forceinline__ void e_load_kv(EIn& in, const uint16_t* k, const uint16_t* v, const ELoc& l, int H, int Hk,
                                          int tid) {
    // value head h reads key head h / (H / Hk); v has H heads
    const uint32_t last = (uint32_t)max(l.rows - 1, 0);
    const uint32_t rs = (uint32_t)H * KD, rsk = (uint32_t)Hk * KD;
    const uint16_t* kb = k + ((size_t)l.tok0 * rsk + (size_t)(l.h / (H / Hk)) * KD);
    const uint16_t* vb = v + ((size_t)l.tok0 * rs + (size_t)l.h * KD);
    const uint32_t R = (uint32_t)min(tid >> 6, C / 16 - 1), d0 = 2u * (uint32_t)(tid & 63);
    const uint32_t r0 = 16u * R;
    const uint32_t ok0 = (r0 * rsk + d0) * 2u, okl = (last * rsk + d0) * 2u;   // k bytes
    const uint32_t ov0 = (r0 * rs + d0) * 2u, ovl = (last * rs + d0) * 2u;     // v bytes
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
        in.k[ii] = *cptr<uint32_t>(kb, min(ok0 + ii * rsk * 2u, okl));
        in.v[ii] = *cptr<uint32_t>(vb, min(ov0 + ii * rs * 2u, ovl));
    }
}

// Issues as many vector-memory operations as phase PQ issues after its next-item loads (N
// stores of zero into the workgroup's pad area), on the paths into an item that do not pass
// through PQ.  Where phase E first uses those loads, the compiler waits with the smallest count
// of younger operations over all paths into the item loop; with this the count includes PQ's
// result stores, so phase E waits for its inputs only, not for the previous item's stores too.
// A lane stores at distinct addresses 16 words apart (no store is merged or dropped, and all
// offsets fit the instruction's immediate field); lanes of the workgroup overlap, all storing
// zero; nothing reads the pad.
constexpr int PAD_WORDS = 1024;  // per workgroup: threads + 16 * (N - 1) words for N <= 32
template <int N, int THREADS>
__device__ __forceinline__ void vm_pad(uint32_t* p) {
    static_assert(THREADS + 16 * (N - 1) <= PAD_WORDS, "pad area");
    // the stores must follow the loads issued before: without this the compiler is free to
    // move them ahead (they touch no input), and then they pad nothing
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) p[16 * i] = 0u;
}

// Exact decayed products of the diagonal tile (R, R) in its wide key dimensions, those whose
// gates are too wide for pivot factors: one exponential per pair and dimension,
// exp(-|gamma_a - gamma_b|), which for g <= 0 is the decay exp(gamma_i - gamma_j) of the pair's
// later row i over its earlier row j.  The other dimensions are left to the pivot products.
// Lane (r16, q4) returns, in the accumulator layouts of phase AA2 (a = 16 R + r16,
// b = 16 R + 4 q4 + e),
//     dA[e] = sum_d k_b k_a decay      (A tile: row b, column a)
//     dQ[e] = sum_d q_a k_b decay      (A2^T tile: row b, column a)
// with the L2 scales of the rows applied (knr for keys, rq for the lane's query row) and rows at
// or past `rows` taken as zero; the caller applies the triangle masks, beta and scale.  gam holds
// phase E's row factors, row stride ld floats: in a wide dimension the log factor against the
// tile's row pivot minus one (<= -1; gamma up to a constant of the tile), in the others the
// factor itself (> 0), which marks them.
template <bool L2N>
__device__ __forceinline__ void diag_exact(const float* gam, int ld, const uint16_t* kbase, const uint16_t* qbase,
                                           uint32_t rsk, int rows, int R, int r16, int q4, const float* knr,
                                           float rq, f32x4& dA, f32x4& dQ) {
    const int a = 16 * R + r16;
    const uint32_t oa = (uint32_t)min(a, rows - 1) * rsk * 2u;
    const float sk = a < rows ? (L2N ? knr[a] : 1.f) : 0.f, sq = a < rows ? rq : 0.f;
    uint32_t ob[4];
    float sb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int b = 16 * R + 4 * q4 + e;
        ob[e] = (uint32_t)min(b, rows - 1) * rsk * 2u;
        sb[e] = b < rows ? (L2N ? knr[b] : 1.f) : 0.f;
        dA[e] = 0.f;
        dQ[e] = 0.f;
    }
    for (int dc = 0; dc < KD / 8; ++dc) {
        // dimensions 8 dc .. 8 dc + 7: only the wide ones (ga < 0, which holds for every row of
        // the tile alike) are summed, the others' operands of row a are zeroed
        const float4* gpa = reinterpret_cast<const float4*>(gam + a * ld + 8 * dc);
        const float4 a0 = gpa[0], a1 = gpa[1];
        const float ga[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        bool any = false;
#pragma unroll
        for (int t = 0; t < 8; ++t) any |= ga[t] < 0.f;
        if (__ballot(any) == 0) continue;
        float ka[8], qa[8];
        unpack8(*cptr<uint4>(kbase, oa + 16u * dc), ka);
        unpack8(*cptr<uint4>(qbase, oa + 16u * dc), qa);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            ka[t] = ga[t] < 0.f ? ka[t] : 0.f;
            qa[t] = ga[t] < 0.f ? qa[t] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float kb[8];
            unpack8(*cptr<uint4>(kbase, ob[e] + 16u * dc), kb);
            const float4* gpb = reinterpret_cast<const float4*>(gam + (16 * R + 4 * q4 + e) * ld + 8 * dc);
            const float4 b0 = gpb[0], b1 = gpb[1];
            const float gb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            float sA = 0.f, sQ = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float kd = kb[t] * ex(-fabsf(ga[t] - gb[t]));   // finite in every column
                sA += kd * ka[t];
                sQ += kd * qa[t];
            }
            dA[e] += sA;
            dQ[e] += sQ;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        dA[e] *= sb[e] * sk;
        dQ[e] *= sb[e] * sq;
    }
}

// One (chunk slot, head) item.  sc is the workgroup's scratch slot; ein holds the item's
// phase E inputs on entry and those of next_item (-1: none) on exit.
template <int C, bool PER_DIM, bool L2N>
__device__ __forceinline__ void intra_item(
    const uint16_t* q, const uint16_t* k, const uint16_t* v,
    const float* g, const float* beta, const ChunkMap& map, int H, int Hk,
    float scale, const Work& ws, unsigned char* smem, int slot, int h, size_t sc, EIn& ein, int next_item,
    uint32_t* pad) {
    using S = IntraShape<C>;
    constexpr int NT = S::NT, NS = S::NS;
    float* Ep = reinterpret_cast<float*>(smem);                                   // [C][EP_LD]
    uint16_t* colh = reinterpret_cast<uint16_t*>(smem + S::R1);                   // [C][COL_LD]
    uint16_t* coll = colh + C * S::COL_LD;
    float* F = reinterpret_cast<float*>(smem + S::R1 + S::R2);                   // [NOFF][KD]
    float* ttot = F;                                                              // [NT][KD], before F
    float* gmid = reinterpret_cast<float*>(smem + S::R1 + S::R2 + S::RF);        // [NT][KD]
    float* egm = gmid + NT * KD;                                                  // [NT][KD]
    float* bet = egm + NT * KD;                                                   // [C]
    float* grow = bet + C;                                                        // [C] per-head gamma
    float* knr = grow + C;                                                        // [C] key row scales
    float* Atile = reinterpret_cast<float*>(smem);                                // after AA2

    // laundered so that the per-thread offsets derived from it are recomputed for every item
    // instead of being hoisted out of the item loop and held in registers across it
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    int64_t tok0;
    int rows;
    slot_chunk(map, slot, tok0, rows);
    if (rows == 0) {
        const ELoc nl = e_locate(map, H, next_item);
        e_load_g<C, PER_DIM>(ein, g, beta, nl, H, tid);
        e_load_kv<C>(ein, k, v, nl, H, Hk, tid);
        vm_pad<S::NPAD, S::THREADS>(pad);
        return;
    }
    const size_t ch = (size_t)slot * H + h;
    // the workgroup's scratch slot
    uint16_t* kgS = ws.kgT + sc * KD * C;
    const int lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    // q and k: key head h / (H / Hk) of Hk; uniform item bases, 32-bit byte offsets per lane
    const uint32_t rsk = (uint32_t)Hk * KD;
    const size_t basek = (size_t)tok0 * rsk + (size_t)(h / (H / Hk)) * KD;
    const uint16_t* kbase = k + basek;
    const uint16_t* qbase = q + basek;

    // Row operands of phase AA2 (raw k and q rows of the wave's two tile rows), loaded
    // before phase E so that their latency is hidden behind it.  The loads are unconditional
    // (rows past the end read the last row) and rows past the end are zeroed after phase E:
    // a load that only some lanes need would be issued under a branch, and the wait count
    // the compiler derives after such a branch covers every load in flight.
    // waves w and w + NT/2 share tile rows cp = w % (NT/2) and NT-1-cp: NT+1 tiles, HF for the
    // first.  The NT active waves are consecutive, so at C = 64 they are spread over the four
    // SIMDs (one each) instead of sharing two.
    const int cp = wave % (NT / 2), part = wave / (NT / 2);
    const bool aa_active = wave < NT;
    const int Rown[2] = {cp, NT - 1 - cp};
    // The second wave of a pair has no tile in the first row (its tiles start at HF > cp), so
    // only the first wave loads that row.  The condition is wave-uniform; phase E's wait counts
    // then follow the shorter path, so the waves that do load also wait for 8 of the previous
    // item's stores, which costs less than the loads saved (measured).
    uint4 kfr[2][KD / 32], qfr[2][KD / 32];
#pragma unroll
    for (int o = 1; o >= 0; --o) {
        const uint32_t ro = ((uint32_t)min(16 * Rown[o] + r16, rows - 1) * rsk + 8u * q4) * 2u;
        const bool need = o == 1 || part == 0;
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks) {
            kfr[o][ks] = need ? *cptr<uint4>(kbase, ro + 64u * ks) : make_uint4(0u, 0u, 0u, 0u);
            qfr[o][ks] = need ? *cptr<uint4>(qbase, ro + 64u * ks) : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    // exp(gamma) k and v of the thread's phase E block as 16-byte fragment slots [hh][c],
    // kept in registers until the A tiles leave LDS, then staged there for the solve
    uint4 xs[2][2], xls[2][2], vs[2][2];  // exp(gamma) k split into high (xs) and low parts
    uint4 kls[2][2];  // low part of kg^T, the two pi-order halves of each slot, to LDS after the solve
    // per-dimension gates too wide for the tile-middle pivots somewhere in the chunk (same value in
    // every thread of the workgroup after phase E's first barrier).  Which (tile, key dimension)
    // columns are wide is kept in LDS as two 64-bit masks per tile, even and odd dimensions.
    bool wide = false;
    uint64_t* wmask = reinterpret_cast<uint64_t*>(grow);   // [NT][2]
    // ------------------------------------------------------------------ phase E
    {
        const int R = tid >> 6, d0 = 2 * (tid & 63);  // tile row R, columns d0, d0 + 1
        const bool act = R < NT;
        float gm2[16][2];
        uint32_t kr[16], vr[16];
        if (tid < C) bet[tid] = (tid < rows) ? ein.b : 0.f;
        if (act) {
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                const bool ok = 16 * R + ii < rows;  // rows past the end are zero
                kr[ii] = ok ? ein.k[ii] : 0u;
                vr[ii] = ok ? ein.v[ii] : 0u;
                gm2[ii][0] = ok ? ein.g[ii].x : 0.f;
                gm2[ii][1] = ok ? ein.g[ii].y : 0.f;
            }
#pragma unroll
            for (int ii = 1; ii < 16; ++ii) {
                gm2[ii][0] += gm2[ii - 1][0];
                gm2[ii][1] += gm2[ii - 1][1];
            }
            *reinterpret_cast<float2*>(ttot + R * KD + d0) = make_float2(gm2[15][0], gm2[15][1]);
            if constexpr (PER_DIM) {
                // per column, the gate span of the tile on either side of its middle row (the
                // exponent of the largest pivot factor); the column is wide above SAFE_SPAN
                bool wc[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float span = 0.f;
#pragma unroll
                    for (int ii = 0; ii < 16; ++ii) span = fmaxf(span, fabsf(gm2[ii][c] - gm2[8][c]));
                    wc[c] = !(span <= SAFE_SPAN);
                }
                const uint64_t m0 = __ballot(wc[0]), m1 = __ballot(wc[1]);
                if ((tid & 63) == 0) {
                    wmask[2 * R] = m0;
                    wmask[2 * R + 1] = m1;
                }
            }
        }
        // in-kernel L2 normalisation of keys: k / sqrt(|k|^2 + eps) per token, the row sum of
        // squares reduced across the wave (the 64 lanes hold the row's 128 columns)
        float rnk[16];
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) rnk[ii] = 1.f;
        if (L2N && act) {
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                const float a = __uint_as_float(kr[ii] << 16), b = __uint_as_float(kr[ii] & 0xffff0000u);
                float ssq = a * a + b * b;
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) ssq += __shfl_xor(ssq, m, 64);
                rnk[ii] = rsqrtf(ssq + L2N_EPS);
            }
            if ((tid & 63) == 0) {
#pragma unroll
                for (int ii = 0; ii < 16; ++ii) knr[16 * R + ii] = rnk[ii];
            }
        }
        lds_barrier();
        if constexpr (PER_DIM) {
#pragma unroll
            for (int Rp = 0; Rp < NT; ++Rp) wide |= (wmask[2 * Rp] | wmask[2 * Rp + 1]) != 0;
        }
        if (act) {
            float off[2] = {0.f, 0.f}, gcl[2] = {0.f, 0.f};
            for (int Rp = 0; Rp < NT; ++Rp) {
                const float2 t = *reinterpret_cast<const float2*>(ttot + Rp * KD + d0);
                if (Rp < R) {
                    off[0] += t.x;
                    off[1] += t.y;
                }
                gcl[0] += t.x;
                gcl[1] += t.y;
            }
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                gm2[ii][0] += off[0];
                gm2[ii][1] += off[1];
            }
            // pivots of the tile, per column: gpr for its rows, gpc for its columns.  Narrow:
            // both the middle row's gamma.  Wide: gamma before the tile's first row (off) for the
            // rows and at its last row for the columns, so that every factor is <= 1 for g <= 0
            // dgc = gpc - gpr: 0 in a narrow column, the tile's total log decay (< -SAFE_SPAN) in a
            // wide one
            float gpr[2], dgc[2], e_gm[2], e_cm[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const bool wcol = PER_DIM && ((wmask[2 * R + c] >> (tid & 63)) & 1u) != 0u;
                const float gpc = wcol ? gm2[15][c] : gm2[8][c];
                gpr[c] = wcol ? off[c] : gm2[8][c];
                dgc[c] = gpc - gpr[c];
                e_gm[c] = ex(gpr[c]);         // exp(gamma at the row pivot) <= 1
                e_cm[c] = ex(gcl[c] - gpc);   // exp(gamma_C - gamma at the column pivot) <= 1
            }
            *reinterpret_cast<float2*>(gmid + R * KD + d0) = make_float2(gpr[0], gpr[1]);
            *reinterpret_cast<float2*>(egm + R * KD + d0) = make_float2(e_gm[0], e_gm[1]);
            if (R == 0) *mptr<float2>(ws.gC + ch * KD, d0 * 4u) = make_float2(ex(gcl[0]), ex(gcl[1]));
            if constexpr (!PER_DIM) {
                if ((tid & 63) == 0) {
#pragma unroll
                    for (int ii = 0; ii < 16; ++ii) grow[16 * R + ii] = gm2[ii][0];
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                // column-major outputs of rows 16R + 8hh .. +7, two bf16 (consecutive rows) per register
                uint32_t bwh[2][4], bwl[2][4], kgh[2][4], kgl[2][4], vtp[2][4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    // kf: the key; fx, fk: its factors exp(gamma_i) (for w; beta enters through
                    // T diag(beta)) and exp(gamma_C - gamma_i) (for kg)
                    float kf[2][2], fx[2][2], fk[2][2];   // [row of the pair][column]
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const int ii = 8 * hh + 2 * e2 + rr;
                        kf[rr][0] = __uint_as_float(kr[ii] << 16) * rnk[ii];
                        kf[rr][1] = __uint_as_float(kr[ii] & 0xffff0000u) * rnk[ii];
                        if constexpr (PER_DIM) {
                            float ep[2], em[2], lg[2];
#pragma unroll
                            for (int c = 0; c < 2; ++c) {
                                lg[c] = gm2[ii][c] - gpr[c];
                                ep[c] = ex(lg[c]);   // exp(gamma_i - row pivot)
                                em[c] = ex(dgc[c] - lg[c]);   // exp(column pivot - gamma_i)
                                fx[rr][c] = e_gm[c] * ep[c];
                                fk[rr][c] = em[c] * e_cm[c];
                            }
                            const int i = 16 * R + ii;
                            // row factors of phase AA2 (> 0); for a wide column instead the log
                            // factor minus one (<= -1), from which AA2 forms the factor and the
                            // diagonal tile the exact pair decays
                            *reinterpret_cast<float2*>(Ep + i * S::EP_LD + d0) =
                                make_float2(dgc[0] < 0.f ? lg[0] - 1.f : ep[0], dgc[1] < 0.f ? lg[1] - 1.f : ep[1]);
                            uint32_t chv, clv;
                            split2(kf[rr][0] * em[0], kf[rr][1] * em[1], chv, clv);
                            *reinterpret_cast<uint32_t*>(colh + i * S::COL_LD + d0) = chv;
                            *reinterpret_cast<uint32_t*>(coll + i * S::COL_LD + d0) = clv;
                        } else {
                            // one gate per token: both factors directly, each <= 1 for g <= 0
                            const float xg = ex(gm2[ii][0]), kgf = ex(gcl[0] - gm2[ii][0]);
#pragma unroll
                            for (int c = 0; c < 2; ++c) {
                                fx[rr][c] = xg;
                                fk[rr][c] = kgf;
                            }
                        }
                    }
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        // exp(gamma_i) k and exp(gamma_C - gamma_i) k
                        split2(kf[0][c] * fx[0][c], kf[1][c] * fx[1][c], bwh[c][e2], bwl[c][e2]);
                        split2(kf[0][c] * fk[0][c], kf[1][c] * fk[1][c], kgh[c][e2], kgl[c][e2]);
                    }
                    const uint32_t v0 = vr[8 * hh + 2 * e2], v1 = vr[8 * hh + 2 * e2 + 1];
                    vtp[0][e2] = (v0 & 0xffffu) | (v1 << 16);
                    vtp[1][e2] = (v0 >> 16) | (v1 & 0xffff0000u);
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    // (K, C) / (V, C) fragment (d / 16, R / 2): rows 16 R + 8 hh .. +7 of column d
                    // are exactly the 16-byte slot of lane (d % 16) + 16 (2 (R % 2) + hh)
                    const int d = d0 + c;
                    // byte offsets inside the workgroup's scratch slot (uniform bases)
                    const uint32_t fo = frag32(d >> 4, R >> 1, C / 32);
                    xs[hh][c] = make_uint4(bwh[c][0], bwh[c][1], bwh[c][2], bwh[c][3]);
                    xls[hh][c] = make_uint4(bwl[c][0], bwl[c][1], bwl[c][2], bwl[c][3]);
                    // kg^T in pi order: rows 16 R + 4 q .. + 3 go to lane (d % 16) + 16 q, half R % 2
                    const uint32_t p0 = (fo + fragP(R & 1, d & 15, 2 * hh)) * 2u, p1 = (fo + fragP(R & 1, d & 15, 2 * hh + 1)) * 2u;
                    *mptr<uint2>(kgS, p0) = make_uint2(kgh[c][0], kgh[c][1]);
                    *mptr<uint2>(kgS, p1) = make_uint2(kgh[c][2], kgh[c][3]);
                    kls[hh][c] = make_uint4(kgl[c][0], kgl[c][1], kgl[c][2], kgl[c][3]);
                    vs[hh][c] = make_uint4(vtp[c][0], vtp[c][1], vtp[c][2], vtp[c][3]);
                }
            }
        }
        lds_barrier();
        if constexpr (PER_DIM) {
            // strictly lower pairs p = R(R-1)/2 + J: F = exp(row pivot of R - column pivot of J) <= 1.
            // The column pivot of J is its row pivot (the middle row's gamma), or in a wide column
            // gamma at its last row: the row pivot plus the log factor that Ep holds there
            for (int e = 4 * tid; e < S::NOFF * KD; e += 4 * S::THREADS) {
                const int p = e / KD, d = e % KD;
                const int R = (int)((1.f + __builtin_sqrtf(8.f * p + 1.f)) * 0.5f);  // R(R-1)/2 <= p < R(R+1)/2
                const int J = p - R * (R - 1) / 2;
                const float4 a = *reinterpret_cast<const float4*>(gmid + R * KD + d);
                float4 b = *reinterpret_cast<const float4*>(gmid + J * KD + d);
                if (wide) {
                    const float4 gl = *reinterpret_cast<const float4*>(Ep + (16 * J + 15) * S::EP_LD + d);
                    b = make_float4(gl.x < 0.f ? b.x + (gl.x + 1.f) : b.x, gl.y < 0.f ? b.y + (gl.y + 1.f) : b.y,
                                    gl.z < 0.f ? b.z + (gl.z + 1.f) : b.z, gl.w < 0.f ? b.w + (gl.w + 1.f) : b.w);
                }
                *reinterpret_cast<float4*>(F + e) = make_float4(ex(a.x - b.x), ex(a.y - b.y), ex(a.z - b.z), ex(a.w - b.w));
            }
        }
    }
    lds_barrier();

    // ------------------------------------------------------------------ phase AA2
#pragma unroll
    for (int o = 0; o < 2; ++o)
        if (16 * Rown[o] + r16 >= rows) {
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks) {
                kfr[o][ks] = make_uint4(0u, 0u, 0u, 0u);
                qfr[o][ks] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    // L2 scales of the wave's own q and k rows: lanes r16 + 16 q4 (q4 = 0..3) share a row
    float rk2[2] = {1.f, 1.f}, rq2[2] = {1.f, 1.f};
    if constexpr (L2N) {
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            // sums of squares straight from the packed bf16 pairs (two products per
            // instruction): unpacking them here would let the compiler keep the unpacked
            // values alive into the tile loop below, which needs them only scaled
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks) {
                const uint4 kv = kfr[o][ks], qv = qfr[o][ks];
                sk = dot2_bf16(kv.x, kv.x, sk);
                sk = dot2_bf16(kv.y, kv.y, sk);
                sk = dot2_bf16(kv.z, kv.z, sk);
                sk = dot2_bf16(kv.w, kv.w, sk);
                sq = dot2_bf16(qv.x, qv.x, sq);
                sq = dot2_bf16(qv.y, qv.y, sq);
                sq = dot2_bf16(qv.z, qv.z, sq);
                sq = dot2_bf16(qv.w, qv.w, sq);
            }
            sk += __shfl_xor(sk, 16, 64);
            sk += __shfl_xor(sk, 32, 64);
            sq += __shfl_xor(sq, 16, 64);
            sq += __shfl_xor(sq, 32, 64);
            rk2[o] = rsqrtf(sk + L2N_EPS);
            rq2[o] = rsqrtf(sq + L2N_EPS);
        }
    }
    // A tiles go to LDS after the phase; the A2 fragments and the qg tile of the wave's
    // diagonal tile stay in registers until phase PQ (no scratch round trip)
    f32x4 accA[S::SMAX];
    uint2 a2keep[S::SMAX];
    uint4 qgkeep[KD / 32];
    f32x4 acc1[S::SMAX], acc2[S::SMAX];
#pragma unroll
    for (int ks = 0; ks < KD / 32; ++ks) qgkeep[ks] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int s = 0; s < S::SMAX; ++s) {
        acc1[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc2[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // the wave's tiles: positions p in [plo, phi) of the row pair's list; p <= cp is tile
    // (cp, p) of the first row, p > cp tile (NT-1-cp, p-cp-1) of the second
    const int plo = part ? S::HF : 0, phi = part ? NT + 1 : S::HF;
    if constexpr (PER_DIM) {
        // Row by row: the row's operands times exp(gamma_i - row pivot of R) (and its L2 scale)
        // are formed once per 32-column step and reused by every tile of the row; a tile
        // below the diagonal multiplies them by F = exp(row pivot of R - column pivot of J) only.
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const bool has = aa_active && (o == 0 ? plo <= cp : phi - 1 > cp);
            if (!has) continue;
            const int R = Rown[o];
            const int i = 16 * R + r16;
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks) {
                const int dd = 32 * ks + 8 * q4;
                float kE[8], qE[8];
                unpack8(kfr[o][ks], kE);
                unpack8(qfr[o][ks], qE);
                {
                    const float4* epp = reinterpret_cast<const float4*>(Ep + i * S::EP_LD + dd);
                    const float4 e0 = epp[0], e1 = epp[1];
                    float ep[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
                    if (wide) {  // a wide column holds the log factor minus one: the factor, <= 1
#pragma unroll
                        for (int e = 0; e < 8; ++e) ep[e] = ep[e] < 0.f ? ex(ep[e] + 1.f) : ep[e];
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        kE[e] *= (L2N ? rk2[o] : 1.f) * ep[e];
                        qE[e] *= (L2N ? rq2[o] : 1.f) * ep[e];
                    }
                }
#pragma unroll
                for (int s = 0; s < S::SMAX; ++s) {
                    const int p = plo + s;
                    if (p >= phi || (p <= cp) != (o == 0)) continue;
                    const int J = (o == 0) ? p : p - cp - 1;
                    const int j = 16 * J + r16;
                    const bf16x8 bhi = as_bf16x8(*reinterpret_cast<const uint4*>(colh + j * S::COL_LD + dd));
                    const bf16x8 blo = as_bf16x8(*reinterpret_cast<const uint4*>(coll + j * S::COL_LD + dd));
                    uint4 ah, al, aq;
                    if (J < R) {
                        const float4* fp = reinterpret_cast<const float4*>(F + (R * (R - 1) / 2 + J) * KD + dd);
                        const float4 f0 = fp[0], f1 = fp[1];
                        const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
                        float rk[8], rq[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            rk[e] = kE[e] * f[e];
                            rq[e] = qE[e] * f[e];
                        }
                        split2(rk[0], rk[1], ah.x, al.x);
                        split2(rk[2], rk[3], ah.y, al.y);
                        split2(rk[4], rk[5], ah.z, al.z);
                        split2(rk[6], rk[7], ah.w, al.w);
                        aq.x = pack_bf2(rq[0], rq[1]);
                        aq.y = pack_bf2(rq[2], rq[3]);
                        aq.z = pack_bf2(rq[4], rq[5]);
                        aq.w = pack_bf2(rq[6], rq[7]);
                    } else {
                        // qg = scale q exp(gamma) = scale (q Ep) exp(gamma_m): (C, K) fragment (R, ks)
                        const float4* gp = reinterpret_cast<const float4*>(egm + R * KD + dd);
                        const float4 g0 = gp[0], g1 = gp[1];
                        const float eg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                        uint4 pq;
                        pq.x = pack_bf2(scale * qE[0] * eg[0], scale * qE[1] * eg[1]);
                        pq.y = pack_bf2(scale * qE[2] * eg[2], scale * qE[3] * eg[3]);
                        pq.z = pack_bf2(scale * qE[4] * eg[4], scale * qE[5] * eg[5]);
                        pq.w = pack_bf2(scale * qE[6] * eg[6], scale * qE[7] * eg[7]);
                        qgkeep[ks] = pq;
                        // in a wide column the pivot product of a pair (i, j) in this tile is its
                        // decay times the tile's total decay, below exp(-SAFE_SPAN): left in, next
                        // to the exact sum of those columns (diag_exact)
                        split2(kE[0], kE[1], ah.x, al.x);
                        split2(kE[2], kE[3], ah.y, al.y);
                        split2(kE[4], kE[5], ah.z, al.z);
                        split2(kE[6], kE[7], ah.w, al.w);
                        aq.x = pack_bf2(qE[0], qE[1]);
                        aq.y = pack_bf2(qE[2], qE[3]);
                        aq.z = pack_bf2(qE[4], qE[5]);
                        aq.w = pack_bf2(qE[6], qE[7]);
                    }
                    const bf16x8 ahi = as_bf16x8(ah), alo = as_bf16x8(al), aqv = as_bf16x8(aq);
                    acc1[s] = mfma32(ahi, bhi, acc1[s]);
                    acc1[s] = mfma32(alo, bhi, acc1[s]);
                    acc1[s] = mfma32(ahi, blo, acc1[s]);
                    acc2[s] = mfma32(bhi, aqv, acc2[s]);   // A2^T tile: rows j, columns i
                }
            }
        }
    }
    // wide columns: the wave's diagonal tile exactly in those columns (their pivot products above
    // are finite but not the pair decays), added to the pivot products of the other columns; tile
    // row cp for the first wave of a pair, NT-1-cp for the second
    f32x4 dA = {0.f, 0.f, 0.f, 0.f}, dQ = dA;
    if (PER_DIM && wide && aa_active) {
        const int Rd = part ? NT - 1 - cp : cp;
        diag_exact<L2N>(Ep, S::EP_LD, kbase, qbase, rsk, rows, Rd, r16, q4, knr,
                        L2N ? (part ? rq2[1] : rq2[0]) : 1.f, dA, dQ);
    }
    if constexpr (!PER_DIM) {
#pragma unroll
        for (int s = 0; s < S::SMAX; ++s) {
            const int p = plo + s;
            if (!aa_active || p >= phi) continue;
            const int o = (p <= cp) ? 0 : 1;
            const int R = Rown[o];
            const int J = (o == 0) ? p : p - cp - 1;
            const int i = 16 * R + r16, j = 16 * J + r16;
            const float rq = o ? rq2[1] : rq2[0];
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks) {
                const int dd = 32 * ks + 8 * q4;
                const uint4 krv = o ? kfr[1][ks] : kfr[0][ks];
                const uint4 qrv = o ? qfr[1][ks] : qfr[0][ks];
                const uint4 kx = *cptr<uint4>(kbase, ((uint32_t)min(j, rows - 1) * rsk + dd) * 2u);
                const bf16x8 b = as_bf16x8((j < rows) ? kx : make_uint4(0, 0, 0, 0));
                if (J == R) {
                    float qf[8];
                    unpack8(qrv, qf);
                    const float f = scale * ex(grow[i]) * rq;
                    uint4 pq;
                    pq.x = pack_bf2(f * qf[0], f * qf[1]);
                    pq.y = pack_bf2(f * qf[2], f * qf[3]);
                    pq.z = pack_bf2(f * qf[4], f * qf[5]);
                    pq.w = pack_bf2(f * qf[6], f * qf[7]);
                    qgkeep[ks] = pq;
                }
                acc1[s] = mfma32(as_bf16x8(krv), b, acc1[s]);
                acc2[s] = mfma32(b, as_bf16x8(qrv), acc2[s]);   // A2^T tile: rows j, columns i
            }
        }
    }
#pragma unroll
    for (int s = 0; s < S::SMAX; ++s) {
        accA[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        a2keep[s] = make_uint2(0u, 0u);
        const int p = plo + s;
        if (!aa_active || p >= phi) continue;
        const int o = (p <= cp) ? 0 : 1;
        const int R = Rown[o];
        const int J = (o == 0) ? p : p - cp - 1;
        const float rq = o ? rq2[1] : rq2[0];
        // A tile: rows i = 16 R + 4 q4 + rr, column j = 16 J + r16
        // A2^T tile: rows j = 16 J + 4 q4 + rr, column i = 16 R + r16
        float a2v[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int ii = 16 * R + 4 * q4 + rr, jj = 16 * J + r16;
            const int i2 = 16 * R + r16, j2 = 16 * J + 4 * q4 + rr;
            float a = acc1[s][rr], a2 = acc2[s][rr];
            if constexpr (PER_DIM) {
                if (wide && J == R) {
                    a += dA[rr];
                    a2 += dQ[rr];
                }
            } else {
                a *= (jj <= ii) ? ex(grow[ii] - grow[jj]) : 0.f;
                a2 *= (j2 <= i2) ? ex(grow[i2] - grow[j2]) : 0.f;
                if constexpr (L2N) {  // raw q, k products: apply the row scales afterwards
                    a *= knr[ii] * knr[jj];
                    a2 *= rq * knr[j2];
                }
            }
            accA[s][rr] = (jj < ii) ? a * bet[ii] : 0.f;
            a2v[rr] = (j2 <= i2) ? a2 * scale : 0.f;
        }
        a2keep[s] = make_uint2(pack_bf2(a2v[0], a2v[1]), pack_bf2(a2v[2], a2v[3]));
    }
    // the global stores of phase E complete before the barrier: from here on the whole
    // workgroup reads them back
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();

    // ------------------------------------------------------------------ phase INV
    // 16-blocks of K (for w) and of V (for u) this wave produces in WU: wave + IW di
    // high part of kg^T for phase PQ from scratch, the same number of fragments per wave; it
    // goes to LDS (R1) after the solve
    constexpr int NKG = 2 * (KD / 16) * NS;  // kg^T fragments in LDS (high, then low)
    constexpr int KPW = NKG / 2 / S::IW;     // high fragments per wave
    static_assert(NKG % (2 * S::IW) == 0, "kg^T fragments per wave");
    static_assert(NKG * 1024 <= S::R1, "kg^T staging");
    u32x4v kgr[KPW];  // a vector type: a struct copy would go through private memory
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int f = wave + S::IW * i;  // fragment (f / NS, f % NS)
        kgr[i] = *cptr<u32x4v>(kgS, (frag32(f / NS, f % NS, C / 32) + lane * 8) * 2u);
    }
    // the gates and beta of the next item (phase E inputs), in flight from here on
    const ELoc nl = e_locate(map, H, next_item);
#pragma unroll
    for (int s = 0; s < S::SMAX; ++s) {
        const int p = (part ? S::HF : 0) + s;
        if (!aa_active || p >= NT + 1 || (part == 0 && s >= S::HF)) continue;
        const int o = (p <= cp) ? 0 : 1;
        const int R = Rown[o];
        const int J = (o == 0) ? p : p - cp - 1;
        tile_store(Atile + tri(R, J) * S::TILE_SZ, accA[s], 1.f, r16, q4, S::TILE_LD);
    }
    lds_barrier();
    // R2 (the column operands of AA2) is free from here on
    float* Tdg = reinterpret_cast<float*>(smem + S::R1);                        // T_RR, fp32 tiles
    uint16_t* Mpre = reinterpret_cast<uint16_t*>(smem + S::R1 + S::TD_BYTES);  // -M_RJ split, J < R
    uint16_t* Tpre = Mpre + S::NOFF * 512;                                      // T'_RR split
    {   // wave R: T_RR = (I + A_RR)^-1, then M_RJ = T_RR A_RJ for J < R and T'_RR = T_RR diag(beta)
        const int R = wave;
        if (R < NT) {
            float* Td = Tdg + R * S::TILE_SZ;
            if (q4 == 0) {  // forward substitution, lane r16 owns column r16
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
#pragma unroll
                for (int ii = 0; ii < 16; ++ii) Td[ii * S::TILE_LD + jc] = t[ii];
            }
            wave_lds_sync();
            // lane (r16, q4): row r16, columns 4 q4 .. + 3 of T_RR, the B operand of
            // M_RJ^T = A_RJ^T T_RR^T on the 16x16x16 instruction
            const float4 tr = *reinterpret_cast<const float4*>(Td + r16 * S::TILE_LD + 4 * q4);
            uint2 bh, bl;
            split2(tr.x, tr.y, bh.x, bl.x);
            split2(tr.z, tr.w, bh.y, bl.y);
            const bf16x4 Bh = __builtin_bit_cast(bf16x4, bh), Bl = __builtin_bit_cast(bf16x4, bl);
            {   // T'_RR: column c of T_RR times beta of chunk row 16 R + c; row r keeps its 16 high
                // parts, then its 16 low parts
                const float* br = bet + 16 * R + 4 * q4;
                uint2 h, l;
                split2(tr.x * br[0], tr.y * br[1], h.x, l.x);
                split2(tr.z * br[2], tr.w * br[3], h.y, l.y);
                *reinterpret_cast<uint2*>(Tpre + R * 512 + r16 * 32 + 4 * q4) = h;
                *reinterpret_cast<uint2*>(Tpre + R * 512 + r16 * 32 + 16 + 4 * q4) = l;
            }
            for (int J = 0; J < R; ++J) {
                // A operand: column r16 of A_RJ, rows 4 q4 .. + 3
                const float* Aj = Atile + tri(R, J) * S::TILE_SZ + 4 * q4 * S::TILE_LD + r16;
                uint2 ah, al;
                split2(Aj[0], Aj[S::TILE_LD], ah.x, al.x);
                split2(Aj[2 * S::TILE_LD], Aj[3 * S::TILE_LD], ah.y, al.y);
                const bf16x4 Ah = __builtin_bit_cast(bf16x4, ah), Al = __builtin_bit_cast(bf16x4, al);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma16(Ah, Bh, acc);
                acc = mfma16(Al, Bh, acc);
                acc = mfma16(Ah, Bl, acc);
                // acc[e] = M_RJ[r16][4 q4 + e]; kept negated, high parts then low parts
                uint2 h, l;
                split2(-acc[0], -acc[1], h.x, l.x);
                split2(-acc[2], -acc[3], h.y, l.y);
                uint16_t* mp = Mpre + (R * (R - 1) / 2 + J) * 512 + r16 * 16 + 4 * q4;
                *reinterpret_cast<uint2*>(mp) = h;
                *reinterpret_cast<uint2*>(mp + 256) = l;
            }
        }
    }
    lds_barrier();

    // ------------------------------------------------------------------ phase WU
    constexpr int NA2 = NT + (NT / 2) * (NT / 2 - 1);  // lower A2 fragments
    // exp(gamma) k and v fragments over the A tiles (R1)
    uint16_t* xL = reinterpret_cast<uint16_t*>(smem);
    uint16_t* vL = xL + KD * C;
    static_assert((KD + VD) * C * 2 <= S::R1, "solve operand staging");
    // the low parts of exp(gamma) k after the solve's own operands (R2 and the free F and pivot areas)
    uint16_t* xlL = reinterpret_cast<uint16_t*>(smem + S::R1 + S::SOLVE_BYTES);
    static_assert(S::SOLVE_BYTES + KD * C * 2 <= S::R2 + S::RF + S::RG, "solve operand staging");
    if ((tid >> 6) < NT) {
        const int R = tid >> 6, d0 = 2 * (tid & 63);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int d = d0 + c;
                const uint32_t o = frag32(d >> 4, R >> 1, C / 32) + ((d & 15) + 16 * (2 * (R & 1) + hh)) * 8;
                *reinterpret_cast<uint4*>(xL + o) = xs[hh][c];
                *reinterpret_cast<uint4*>(xlL + o) = xls[hh][c];
                *reinterpret_cast<uint4*>(vL + o) = vs[hh][c];
            }
    }
    lds_barrier();
    // the gates and beta of the next item (phase E inputs), in flight from here on
    e_load_g<C, PER_DIM>(ein, g, beta, nl, H, tid);
    // Blocked forward substitution for [w | u] = (I + A)^-1 diag(beta) [exp(gamma) k | v], wave
    // producing columns 16 dt .. + 15 of each (dt = wave + IW di):
    //     Z_R = T'_RR Y_R - sum_{J<R} M_RJ Z_J.
    // The Z tiles stay in registers, split, in the D layout (lane (r16, q4), element e: row
    // 16 R + 4 q4 + e, column 16 dt + r16), which two at a time are the pi-order B operand of
    // the 16x16x32 instruction.
    uint2 wzh[S::DTW][NT], wzl[S::DTW][NT], uzh[S::DTW][NT], uzl[S::DTW][NT];
#pragma unroll
    for (int R = 0; R < NT; ++R)
#pragma unroll
    for (int di = 0; di < S::DTW; ++di) {
        const int dt = wave + S::IW * di;
        f32x4 aw = {0.f, 0.f, 0.f, 0.f}, au = aw;
        {   // T'_RR Y_R (Y = exp(gamma) k split, v exact in bf16): Y rows 32 (R / 2) + 8 q4 + i in
            // the normal-order fragment R / 2
            uint4 th = make_uint4(0u, 0u, 0u, 0u), tl = th;
            if ((q4 >> 1) == (R & 1)) {
                const uint4* tp = reinterpret_cast<const uint4*>(Tpre + R * 512 + r16 * 32);
                th = tp[q4 & 1];
                tl = tp[2 + (q4 & 1)];
            }
            const bf16x8 thi = as_bf16x8(th), tlo = as_bf16x8(tl);
            const uint32_t fo = frag32(dt, R >> 1, C / 32) + lane * 8;
            const bf16x8 xf = as_bf16x8(*reinterpret_cast<const uint4*>(xL + fo));
            const bf16x8 xlf = as_bf16x8(*reinterpret_cast<const uint4*>(xlL + fo));
            const bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint4*>(vL + fo));
            aw = mfma32(thi, xf, aw);
            aw = mfma32(tlo, xf, aw);
            aw = mfma32(thi, xlf, aw);
            au = mfma32(thi, vf, au);
            au = mfma32(tlo, vf, au);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (2 * s >= R) break;
            // pi-order pair (2 s, 2 s + 1); the second half is zero when 2 s + 1 = R
            const bool two = 2 * s + 1 < R;
            const uint16_t* m0 = Mpre + (R * (R - 1) / 2 + 2 * s) * 512 + r16 * 16 + 4 * q4;
            const uint2 z2 = make_uint2(0u, 0u);
            const uint2 mh0 = *reinterpret_cast<const uint2*>(m0);
            const uint2 ml0 = *reinterpret_cast<const uint2*>(m0 + 256);
            const uint2 mh1 = two ? *reinterpret_cast<const uint2*>(m0 + 512) : z2;
            const uint2 ml1 = two ? *reinterpret_cast<const uint2*>(m0 + 768) : z2;
            const bf16x8 Mh = as_bf16x8(make_uint4(mh0.x, mh0.y, mh1.x, mh1.y));
            const bf16x8 Ml = as_bf16x8(make_uint4(ml0.x, ml0.y, ml1.x, ml1.y));
            const uint2 wh1 = two ? wzh[di][2 * s + 1] : z2, wl1 = two ? wzl[di][2 * s + 1] : z2;
            const uint2 uh1 = two ? uzh[di][2 * s + 1] : z2, ul1 = two ? uzl[di][2 * s + 1] : z2;
            const bf16x8 Zwh = as_bf16x8(make_uint4(wzh[di][2 * s].x, wzh[di][2 * s].y, wh1.x, wh1.y));
            const bf16x8 Zwl = as_bf16x8(make_uint4(wzl[di][2 * s].x, wzl[di][2 * s].y, wl1.x, wl1.y));
            const bf16x8 Zuh = as_bf16x8(make_uint4(uzh[di][2 * s].x, uzh[di][2 * s].y, uh1.x, uh1.y));
            const bf16x8 Zul = as_bf16x8(make_uint4(uzl[di][2 * s].x, uzl[di][2 * s].y, ul1.x, ul1.y));
            aw = mfma32(Mh, Zwh, aw);
            aw = mfma32(Ml, Zwh, aw);
            aw = mfma32(Mh, Zwl, aw);
            au = mfma32(Mh, Zuh, au);
            au = mfma32(Ml, Zuh, au);
            au = mfma32(Mh, Zul, au);
        }
        split2(aw[0], aw[1], wzh[di][R].x, wzl[di][R].x);
        split2(aw[2], aw[3], wzh[di][R].y, wzl[di][R].y);
        split2(au[0], au[1], uzh[di][R].x, uzl[di][R].x);
        split2(au[2], au[3], uzh[di][R].y, uzl[di][R].y);
    }

    // ------------------------------------------------------------------ phase PQ
    // k and v of the next item (the rest of its phase E inputs), in flight through PQ (nothing
    // below waits on the vector memory counter before the next item uses them)
    e_load_kv<C>(ein, k, v, nl, H, Hk, tid);
    lds_barrier();  // every wave is done with the solve operands in R2
    // kg^T to R1 (high part from scratch, low part kept since phase E); the A2 fragments and
    // qg tiles kept since phase AA2 to R2
    uint16_t* kgL = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < KPW; ++i)
        *reinterpret_cast<u32x4v*>(kgL + (wave + S::IW * i) * 512 + lane * 8) = kgr[i];
    if ((tid >> 6) < NT) {
        const int R = tid >> 6, d0 = 2 * (tid & 63);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int d = d0 + c;
                uint16_t* fl = kgL + (NKG / 2) * 512 + frag32(d >> 4, R >> 1, C / 32);
                *reinterpret_cast<uint2*>(fl + fragP(R & 1, d & 15, 2 * hh)) = make_uint2(kls[hh][c].x, kls[hh][c].y);
                *reinterpret_cast<uint2*>(fl + fragP(R & 1, d & 15, 2 * hh + 1)) = make_uint2(kls[hh][c].z, kls[hh][c].w);
            }
    }
    uint16_t* a2L = reinterpret_cast<uint16_t*>(smem + S::R1);  // lower A2 fragments, pi order
    uint16_t* qgL = a2L + NA2 * 512;                             // (qg)^T D tiles
    static_assert(NA2 * 1024 + C * KD * 2 <= S::R2, "A2 and qg staging");
#pragma unroll
    for (int s = 0; s < S::SMAX; ++s) {
        const int p = (part ? S::HF : 0) + s;
        if (!aa_active || p >= NT + 1 || (part == 0 && s >= S::HF)) continue;
        const int o = (p <= cp) ? 0 : 1;
        const int R = Rown[o];
        const int J = (o == 0) ? p : p - cp - 1;
        uint16_t* f = a2L + a2_slot(R, J >> 1) * 512;
        *reinterpret_cast<uint2*>(f + fragP(J & 1, r16, q4)) = a2keep[s];
        // tile (R, R + 1) shares the fragment of an even diagonal tile and is zero
        if (J == R && (R & 1) == 0) *reinterpret_cast<uint2*>(f + fragP(1, r16, q4)) = make_uint2(0u, 0u);
    }
    if (aa_active) {  // each active wave owns one diagonal tile: tile row cp (first part) or NT-1-cp
        const int Rd = part ? NT - 1 - cp : cp;
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks) store_qg(qgL, Rd, ks, r16, q4, qgkeep[ks]);
    }
    // w and u as pi-order operands: tiles 2s and 2s+1 give the 32 contracted rows of step s.
    // Both keep their split for P and B; Q and U take the high parts.
    uint4 wh[S::DTW][NS], wl[S::DTW][NS], uh[S::DTW][NS], ul[S::DTW][NS];
#pragma unroll
    for (int di = 0; di < S::DTW; ++di)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        wh[di][s] = make_uint4(wzh[di][2 * s].x, wzh[di][2 * s].y, wzh[di][2 * s + 1].x, wzh[di][2 * s + 1].y);
        wl[di][s] = make_uint4(wzl[di][2 * s].x, wzl[di][2 * s].y, wzl[di][2 * s + 1].x, wzl[di][2 * s + 1].y);
        uh[di][s] = make_uint4(uzh[di][2 * s].x, uzh[di][2 * s].y, uzh[di][2 * s + 1].x, uzh[di][2 * s + 1].y);
        ul[di][s] = make_uint4(uzl[di][2 * s].x, uzl[di][2 * s].y, uzl[di][2 * s + 1].x, uzl[di][2 * s + 1].y);
    }
    lds_barrier();  // staged kg^T, A2 and qg are in LDS
    uint2 qgv[S::DTW][NT];    // (qg)^T tiles (I, dt)
#pragma unroll
    for (int di = 0; di < S::DTW; ++di)
#pragma unroll
    for (int I = 0; I < NT; ++I)
        qgv[di][I] = *reinterpret_cast<const uint2*>(qgL + ((I * (KD / 16) + wave + S::IW * di) * 64 + lane) * 4);
    // P^T tile (rows d in block dt, columns k in block x) = w^T kg; B tile (rows k in x,
    // columns v in dt) = kg^T u.  -P goes out in pi order as the A operand of -P S.
    // Outputs of the item through uniform bases and 32-bit byte offsets.
    uint16_t* PnI = ws.Pn + ch * 2 * KD * KD;
    float* BmI = ws.Bm + ch * KD * VD;
    uint16_t* QpI = ws.Qp + ch * C * KD;
    uint16_t* UpI = ws.Up + ch * C * VD;
#pragma unroll
    for (int x = 0; x < KD / 16; ++x)
#pragma unroll
    for (int di = 0; di < S::DTW; ++di) {
        const int dt = wave + S::IW * di;
        // P and B from split operands (three MFMAs each): the state goes through P in every
        // chunk, so a single bf16 rounding of w or kg grows into its error where it persists
        f32x4 pt = {0.f, 0.f, 0.f, 0.f}, p1 = pt, b0 = pt, b1 = pt;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const bf16x8 kh = as_bf16x8(*reinterpret_cast<const uint4*>(kgL + (x * NS + s) * 512 + lane * 8));
            const bf16x8 kl = as_bf16x8(*reinterpret_cast<const uint4*>(kgL + (NKG / 2 + x * NS + s) * 512 + lane * 8));
            pt = mfma32(as_bf16x8(wh[di][s]), kh, pt);
            p1 = mfma32(as_bf16x8(wl[di][s]), kh, p1);
            p1 = mfma32(as_bf16x8(wh[di][s]), kl, p1);
            b0 = mfma32(kh, as_bf16x8(uh[di][s]), b0);
            b1 = mfma32(kl, as_bf16x8(uh[di][s]), b1);
            b1 = mfma32(kh, as_bf16x8(ul[di][s]), b1);
        }
        f32x4 bt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bt[e] = b0[e] + b1[e];
            pt[e] += p1[e];
        }
        // -P split into bf16 high and low parts, for the same reason
        uint2 ph, pl;
        split2(-pt[0], -pt[1], ph.x, pl.x);
        split2(-pt[2], -pt[3], ph.y, pl.y);
        const uint32_t po = (frag32(x, dt >> 1, KD / 32) + fragP(dt & 1, r16, q4)) * 2u;
        *mptr<uint2>(PnI, po) = ph;
        *mptr<uint2>(PnI, po + KD * KD * 2u) = pl;
        *mptr<float4>(BmI, ((x * (VD / 16) + dt) * 64 + lane) * 16u) = make_float4(bt[0], bt[1], bt[2], bt[3]);
    }
    // Q^T tile (rows d in dt, columns i in I) = (qg)^T - w^T A2^T; U^T tile (rows v in dt,
    // columns i in I) = u^T A2^T.  A2 fragment (I, s) is the B operand of both.
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int di = 0; di < S::DTW; ++di) {
        const int dt = wave + S::IW * di;
        const uint2 qv = qgv[di][I];
        f32x4 qt = {__uint_as_float(qv.x << 16), __uint_as_float(qv.x & 0xffff0000u), __uint_as_float(qv.y << 16),
                    __uint_as_float(qv.y & 0xffff0000u)};
        f32x4 ut = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (2 * s > I) break;
            const bf16x8 a2 = as_bf16x8(*reinterpret_cast<const uint4*>(a2L + a2_slot(I, s) * 512 + lane * 8));
            qt = mfma32(as_bf16x8(neg_bf16x8(wh[di][s])), a2, qt);
            ut = mfma32(as_bf16x8(uh[di][s]), a2, ut);
        }
        // Q and U are read only by the output kernel, after the chain: streamed past the caches,
        // so that they do not displace -P and B, which the chain reads next.  A Q^T fragment is
        // stored half-major (the 16-row half of tile dt is one contiguous 512-byte block), so each
        // of these stores writes whole cache lines; in pi order two waves would each write half
        // of every line, and lines that bypass the caches are not merged
        st_nt(mptr<uint2>(QpI, (frag32(I, dt >> 1, KD / 32) + (dt & 1) * 256u + lane * 4u) * 2u),
              make_uint2(pack_bf2(qt[0], qt[1]), pack_bf2(qt[2], qt[3])));
        st_nt(mptr<uint2>(UpI, ((I * (VD / 16) + dt) * 64 + lane) * 8u), make_uint2(pack_bf2(ut[0], ut[1]), pack_bf2(ut[2], ut[3])));
    }
}

// Persistent: workgroup b takes items b, b + gridDim.x, ... (item = slot * H + head) and
// keeps its scratch in slot b, so the scratch of all workgroups stays cache-resident.
template <int C, bool PER_DIM, bool L2N>
__global__ __launch_bounds__(IntraShape<C>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void intra_kernel(
    const uint16_t* q, const uint16_t* k, const uint16_t* v,
    const float* g, const float* beta, ChunkMap map, int H, int Hk,
    float scale, Work ws, int nitems, uint32_t* pad_all) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[IntraShape<C>::BYTES];
    uint32_t* pad = pad_all + blockIdx.x * PAD_WORDS + threadIdx.x;
    EIn ein;
    {
        const ELoc l0 = e_locate(map, H, blockIdx.x < nitems ? (int)blockIdx.x : -1);
        e_load_g<C, PER_DIM>(ein, g, beta, l0, H, threadIdx.x);
        e_load_kv<C>(ein, k, v, l0, H, Hk, threadIdx.x);
    }
    vm_pad<IntraShape<C>::NPAD, IntraShape<C>::THREADS>(pad);
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
        // the previous item is done with LDS.  An LDS-only barrier: __syncthreads() would also
        // wait for every load and store in flight (this item's inputs, prefetched during the
        // previous item, and the previous item's results); the only global data read back
        // across waves, the kg^T scratch, is ordered by the wait at the end of phase AA2
        lds_barrier();
        const int next = item + (int)gridDim.x < nitems ? item + (int)gridDim.x : -1;
        intra_item<C, PER_DIM, L2N>(q, k, v, g, beta, map, H, Hk, scale, ws, smem, item / H, item % H,
                               blockIdx.x, ein, next, pad);
    }
}

// Workgroups of this kernel that the current device holds at once (cached per device).
template <int C, bool PER_DIM, bool L2N>
static int resident_groups() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int ncu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, intra_kernel<C, PER_DIM, L2N>, IntraShape<C>::THREADS, 0) !=
            hipSuccess)
        return 1;
    const int r = max(1, ncu * per_cu);
    if (dev >= 0 && dev < 64) cache[dev].store(r, std::memory_order_relaxed);
    return r;
}

template <int C, bool PER_DIM, bool L2N>
static hipError_t launch_intra_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                                 const float* beta, const ChunkMap& map, int nslots, int H, int Hk,
                                 float scale, const Work& ws, int nscratch, hipStream_t stream) {
    const int nitems = nslots * H;
    const int grid = min(min(nitems, nscratch), resident_groups<C, PER_DIM, L2N>());
    // the pad areas of the scratch slots, after the kg^T planes
    uint32_t* pad = reinterpret_cast<uint32_t*>(ws.kgT + (size_t)nscratch * KD * C);
    hipLaunchKernelGGL((intra_kernel<C, PER_DIM, L2N>), dim3(grid), dim3(IntraShape<C>::THREADS), 0, stream, q, k, v, g,
                       beta, map,
                       H, Hk, scale, ws, nitems, pad);
    return hipGetLastError();
}

template <int C, bool PER_DIM>
static hipError_t launch_intra_n(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                                 const float* beta, const ChunkMap& map, int nslots, int H, int Hk, int l2n,
                                 float scale, const Work& ws, int nscratch, hipStream_t stream) {
    return l2n ? launch_intra_t<C, PER_DIM, true>(q, k, v, g, beta, map, nslots, H, Hk, scale, ws, nscratch, stream)
               : launch_intra_t<C, PER_DIM, false>(q, k, v, g, beta, map, nslots, H, Hk, scale, ws, nscratch, stream);
}

hipError_t launch_intra(int C, bool per_dim, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* g, const float* beta, const ChunkMap& map, int nslots, int H, int Hk,
                        int l2n, float scale, const Work& ws, int nscratch, hipStream_t stream) {
    if (C == 64)
        return per_dim ? launch_intra_n<64, true>(q, k, v, g, beta, map, nslots, H, Hk, l2n, scale, ws, nscratch, stream)
                       : launch_intra_n<64, false>(q, k, v, g, beta, map, nslots, H, Hk, l2n, scale, ws, nscratch, stream);
    return per_dim ? launch_intra_n<128, true>(q, k, v, g, beta, map, nslots, H, Hk, l2n, scale, ws, nscratch, stream)
                   : launch_intra_n<128, false>(q, k, v, g, beta, map, nslots, H, Hk, l2n, scale, ws, nscratch, stream);
}

}  // namespace cdr
