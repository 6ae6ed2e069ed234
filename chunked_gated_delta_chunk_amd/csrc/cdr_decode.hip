// Per-token (recurrent) forward of the gated delta rule: the decode path.
//
// The update rule of the page "PyPTO-Gym 的 chunk_kda 算子实战" (section 算子定位与算法背景),
// token by token, on an fp32 state stored as [V, K] (the page's [H, V, K] state per head), as
// the decode-side operator of section 与其他 KDA 算子的关系 does, with the state optionally kept
// in place in a pool addressed by slot indices and with speculative-decoding slots.
//
// Row v of the state only ever meets row v: with s = S[v, :] (length K),
//     s <- s * exp(g)                 (per key dimension, or one scalar per head)
//     s <- s + k * beta (v_v - s . k)
//     o_v = scale * (s . q)
// so the state's rows are independent and a workgroup owns 32 of them for the whole
// sequence, in registers.  Eight lanes share a row group of two rows (16 columns each, as
// four 16-byte pieces 32 columns apart, so that every load and store instruction covers whole
// 128-byte lines), and the dot products per token are 3-step butterflies across those eight
// lanes.  The kernel is bound by streaming the state (64 KiB in and 64 KiB out per sequence and
// head, plus 64 KiB per stored draft position); state traffic uses non-temporal loads and
// stores, since nothing reads a state twice within a call.
#include "chunk_dr.h"
#include "cdr_common.h"

namespace cdr {

namespace {

constexpr int DROWS = 32;                 // state rows per workgroup
constexpr int DRPL = 2;                   // rows per group of eight lanes
constexpr int DTHREADS = DROWS / DRPL * 8;
constexpr int DBLOCKS = VD / DROWS;       // workgroups per (sequence, value head)
constexpr float DEC_L2N_EPS = 1e-6f;      // x / sqrt(|x|^2 + eps)

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    const float* beta;
    const int32_t* cu;       // packed sequence offsets, or null (N rows of T tokens)
    const float* s_in;       // separate states [N, HV, V, K] (may be null), or the pool
    float* s_out;            // separate final states (may be null), or the pool
    const int32_t* idx;      // pool slot indices [N] or [N, L]
    const int32_t* acc;      // accepted-token counts [N], or null (1)
    uint16_t* o;
    int T, H, HV, N;
    int num_slots, L;        // pool size; index columns (0: one slot per sequence)
    int pool;                // states live in the pool
    float scale;
};

// one token's inputs for a lane: its 16 columns of q, k (bf16) and g, beta, v of its rows
struct TokIn {
    uint2 q[4], k[4];
    float4 g[4];
    float b, v[DRPL];
};

template <bool PER_DIM>
__device__ __forceinline__ void tok_load(TokIn& in, const DecodeArgs& a, int64_t tok, int hv, int hk, int row0,
                                         int c0) {
    const size_t qk = ((size_t)tok * a.H + hk) * KD + c0;
    const size_t vh = (size_t)tok * a.HV + hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        in.q[i] = *reinterpret_cast<const uint2*>(a.q + qk + 32 * i);
        in.k[i] = *reinterpret_cast<const uint2*>(a.k + qk + 32 * i);
        if constexpr (PER_DIM) in.g[i] = *reinterpret_cast<const float4*>(a.g + vh * KD + c0 + 32 * i);
    }
    if constexpr (!PER_DIM) in.g[0].x = a.g[vh];
    in.b = a.beta[vh];
#pragma unroll
    for (int r = 0; r < DRPL; ++r) in.v[r] = bf2f(a.v[vh * VD + row0 + r]);
}

__device__ __forceinline__ void unpack4(const uint2& p, float* f) {
    f[0] = __uint_as_float(p.x << 16);
    f[1] = __uint_as_float(p.x & 0xffff0000u);
    f[2] = __uint_as_float(p.y << 16);
    f[3] = __uint_as_float(p.y & 0xffff0000u);
}

// sum over the eight lanes of a row group (lanes 8r .. 8r+7 of the wave)
__device__ __forceinline__ float row_sum(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    return x;
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_rows(float4 (&s)[DRPL][4], const float* base) {
#pragma unroll
    for (int r = 0; r < DRPL; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(base + r * KD + 32 * i));
            s[r][i] = make_float4(x.x, x.y, x.z, x.w);
        }
}

__device__ __forceinline__ void store_rows(float* base, const float4 (&s)[DRPL][4]) {
#pragma unroll
    for (int r = 0; r < DRPL; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4v x = {s[r][i].x, s[r][i].y, s[r][i].z, s[r][i].w};
            __builtin_nontemporal_store(x, reinterpret_cast<f32x4v*>(base + r * KD + 32 * i));
        }
}

template <bool PER_DIM, bool L2N>
__global__ __launch_bounds__(DTHREADS) void decode_kernel(DecodeArgs a) {
    const int blk = blockIdx.x;
    const int rb = blk % DBLOCKS;
    const int hv = (blk / DBLOCKS) % a.HV;
    const int n = blk / (DBLOCKS * a.HV);
    const int tid = threadIdx.x;
    const int row0 = DROWS * rb + DRPL * (tid >> 3);
    const int c0 = 4 * (tid & 7);
    const int hk = hv / (a.HV / a.H);

    int64_t bos;
    int len;
    if (a.cu) {
        bos = a.cu[n];
        len = a.cu[n + 1] - a.cu[n];
    } else {
        bos = (int64_t)n * a.T;
        len = a.T;
    }
    const size_t state = (size_t)VD * KD;
    const size_t in_row = (size_t)row0 * KD + c0;

    // start state
    int slot = -1;
    if (a.pool) {
        if (a.L == 0) {
            slot = a.idx[n];
        } else {
            const int acc = a.acc ? a.acc[n] : 1;
            slot = (acc >= 1 && acc <= a.L) ? a.idx[(size_t)n * a.L + acc - 1] : -1;
        }
        if (slot < 0 || slot >= a.num_slots) {
            // padding entry: zero outputs, no state touched
            if ((tid & 7) == 0)
                for (int t = 0; t < len; ++t)
#pragma unroll
                    for (int r = 0; r < DRPL; ++r) a.o[((size_t)(bos + t) * a.HV + hv) * VD + row0 + r] = 0;
            return;
        }
    }
    float4 s[DRPL][4];
    if (a.pool) {
        load_rows(s, a.s_in + ((size_t)slot * a.HV + hv) * state + in_row);
    } else if (a.s_in) {
        load_rows(s, a.s_in + ((size_t)n * a.HV + hv) * state + in_row);
    } else {
#pragma unroll
        for (int r = 0; r < DRPL; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[r][i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int t = 0; t < len; ++t) {
        const int64_t tok = bos + t;
        TokIn in;
        tok_load<PER_DIM>(in, a, tok, hv, hk, row0, c0);
        // q and k enter through their L2 scales: s.k = rk (s.k_raw), s.q = rq (s.q_raw)
        float rq = 1.f, rk = 1.f;
        if constexpr (L2N) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float qf[4], kf[4];
                unpack4(in.q[i], qf);
                unpack4(in.k[i], kf);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sq += qf[e] * qf[e];
                    sk += kf[e] * kf[e];
                }
            }
            rq = rsqrtf(row_sum(sq) + DEC_L2N_EPS);
            rk = rsqrtf(row_sum(sk) + DEC_L2N_EPS);
        }
        // decay, then the read s . k on the decayed state
        float dot[DRPL];
#pragma unroll
        for (int r = 0; r < DRPL; ++r) dot[r] = 0.f;
        const float dh = PER_DIM ? 0.f : ex(in.g[0].x);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float kf[4];
            unpack4(in.k[i], kf);
            float d[4];
            if constexpr (PER_DIM) {
                d[0] = ex(in.g[i].x);
                d[1] = ex(in.g[i].y);
                d[2] = ex(in.g[i].z);
                d[3] = ex(in.g[i].w);
            } else {
                d[0] = d[1] = d[2] = d[3] = dh;
            }
#pragma unroll
            for (int r = 0; r < DRPL; ++r) {
                float* x = reinterpret_cast<float*>(&s[r][i]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] *= d[e];
                    dot[r] += x[e] * kf[e];
                }
            }
        }
        // s += k beta (v - s . k), then o = scale s . q
        float u[DRPL], so[DRPL];
#pragma unroll
        for (int r = 0; r < DRPL; ++r) {
            u[r] = in.b * (in.v[r] - rk * row_sum(dot[r])) * rk;
            so[r] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float qf[4], kf[4];
            unpack4(in.q[i], qf);
            unpack4(in.k[i], kf);
#pragma unroll
            for (int r = 0; r < DRPL; ++r) {
                float* x = reinterpret_cast<float*>(&s[r][i]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] += kf[e] * u[r];
                    so[r] += x[e] * qf[e];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < DRPL; ++r) {
            const float ov = a.scale * rq * row_sum(so[r]);
            if ((tid & 7) == 0) a.o[((size_t)tok * a.HV + hv) * VD + row0 + r] = f2bf(ov);
        }
        if (a.pool && a.L > 0 && t < a.L) {
            const int w = a.idx[(size_t)n * a.L + t];
            if (w >= 0 && w < a.num_slots) store_rows(a.s_out + ((size_t)w * a.HV + hv) * state + in_row, s);
        }
    }
    if (a.pool) {
        if (a.L == 0) store_rows(a.s_out + ((size_t)slot * a.HV + hv) * state + in_row, s);
    } else if (a.s_out) {
        store_rows(a.s_out + ((size_t)n * a.HV + hv) * state + in_row, s);
    }
}

template <bool PER_DIM>
hipError_t launch_decode_t(const DecodeArgs& a, bool l2n, hipStream_t stream) {
    const dim3 grid((unsigned)((size_t)a.N * a.HV * DBLOCKS));
    if (l2n)
        hipLaunchKernelGGL((decode_kernel<PER_DIM, true>), grid, dim3(DTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<PER_DIM, false>), grid, dim3(DTHREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

}  // namespace cdr

extern "C" {

cdr_status cdr_recurrent_check(const cdr_recurrent_problem* p) {
    if (p == nullptr) return CDR_ERR_NULL_ARG;
    if (p->B <= 0 || p->T < 0 || p->H <= 0 || p->HV < 0 || p->N <= 0 || p->K <= 0 || p->V <= 0)
        return CDR_ERR_BAD_SHAPE;
    const int64_t HV = p->HV > 0 ? p->HV : p->H;
    if (HV % p->H != 0) return CDR_ERR_BAD_SHAPE;
    if (p->K != cdr::KD || p->V != cdr::VD) return CDR_ERR_UNSUPPORTED;
    if (p->gate != CDR_GATE_PER_DIM && p->gate != CDR_GATE_PER_HEAD) return CDR_ERR_UNSUPPORTED;
    if (p->state_mode != CDR_STATE_SEPARATE && p->state_mode != CDR_STATE_POOL &&
        p->state_mode != CDR_STATE_POOL_SPEC)
        return CDR_ERR_UNSUPPORTED;
    if (p->state_mode != CDR_STATE_SEPARATE && p->num_slots <= 0) return CDR_ERR_BAD_SHAPE;
    if (p->state_mode == CDR_STATE_POOL_SPEC && p->index_cols <= 0) return CDR_ERR_BAD_SHAPE;
    if (p->varlen) {
        if (p->B != 1) return CDR_ERR_VARLEN_BATCH;
    } else if (p->N != p->B) {
        return CDR_ERR_BAD_SHAPE;
    }
    if ((int64_t)p->B * p->T > INT32_MAX) return CDR_ERR_BAD_SHAPE;
    if ((int64_t)p->N * HV * cdr::DBLOCKS > INT32_MAX) return CDR_ERR_BAD_SHAPE;
    return CDR_OK;
}

cdr_status chunk_dr_recurrent_fwd(const cdr_recurrent_problem* p, const void* q, const void* k, const void* v,
                                  const float* g, const float* beta, const int32_t* cu_seqlens,
                                  const float* initial_state, float* final_state, float* state_pool,
                                  const int32_t* ssm_state_indices, const int32_t* num_accepted_tokens, void* o,
                                  void* stream) {
    const cdr_status st = cdr_recurrent_check(p);
    if (st != CDR_OK) return st;
    const int64_t tokens = (int64_t)p->B * p->T;
    if (tokens > 0 && (!q || !k || !v || !g || !beta || !o)) return CDR_ERR_NULL_ARG;
    if (p->varlen && !cu_seqlens) return CDR_ERR_NULL_ARG;
    cdr::DecodeArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.g = g;
    a.beta = beta;
    a.cu = p->varlen ? cu_seqlens : nullptr;
    a.o = static_cast<uint16_t*>(o);
    a.T = p->T;
    a.H = p->H;
    a.HV = p->HV > 0 ? p->HV : p->H;
    a.N = p->N;
    a.scale = p->scale;
    a.acc = nullptr;
    a.idx = nullptr;
    a.num_slots = 0;
    a.L = 0;
    if (p->state_mode == CDR_STATE_SEPARATE) {
        if (p->has_initial_state && !initial_state) return CDR_ERR_NULL_ARG;
        if (p->output_final_state && !final_state) return CDR_ERR_NULL_ARG;
        a.pool = 0;
        a.s_in = p->has_initial_state ? initial_state : nullptr;
        a.s_out = p->output_final_state ? final_state : nullptr;
    } else {
        if (!state_pool || !ssm_state_indices) return CDR_ERR_NULL_ARG;
        a.pool = 1;
        a.s_in = state_pool;
        a.s_out = state_pool;
        a.idx = ssm_state_indices;
        a.num_slots = p->num_slots;
        if (p->state_mode == CDR_STATE_POOL_SPEC) {
            a.L = p->index_cols;
            a.acc = num_accepted_tokens;  // null: every sequence starts from column 0
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = p->gate == CDR_GATE_PER_DIM ? cdr::launch_decode_t<true>(a, p->qk_l2norm != 0, s)
                                                     : cdr::launch_decode_t<false>(a, p->qk_l2norm != 0, s);
    return e == hipSuccess ? CDR_OK : CDR_ERR_HIP;
}

}  // extern "C"
