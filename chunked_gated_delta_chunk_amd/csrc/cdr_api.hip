// C interface: validation, workspace layout and kernel launches (declared in chunk_dr.h).
#include "chunk_dr.h"
#include "cdr_common.h"

namespace cdr {
hipError_t launch_intra(int C, bool per_dim, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* g, const float* beta, const ChunkMap& map, int nslots, int H, int Hk,
                        int l2n, float scale, const Work& ws, int nscratch, hipStream_t stream);
hipError_t launch_chain(const ChunkMap& map, int N, int H, const float* s0, float* s_out, const Work& ws,
                        int32_t* order_ws, hipStream_t stream);
hipError_t launch_output(int C, const ChunkMap& map, int nslots, int H, uint16_t* o, const Work& ws,
                         hipStream_t stream);
hipError_t launch_chain_map(const ChunkMap& map, int N, int H, float* m_out, const Work& ws, int32_t* order_ws,
                            hipStream_t stream);
hipError_t launch_merge(int R, int HV, const float* M, const float* X, const float* s0, float* s_in,
                        hipStream_t stream);
}  // namespace cdr

#include "cdr_bwd_api.h"

namespace {

constexpr size_t kAlign = 256;

// value heads (the state, v, g, beta and o carry them); q and k have p->H
int64_t value_heads(const cdr_problem* p) { return p->HV > 0 ? p->HV : p->H; }

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// chunk slots: fixed length B * ceil(T / C); varlen floor(T / C) + N (see ChunkMap)
int64_t num_slots(const cdr_problem* p) {
    if (p->varlen) return (int64_t)p->T / p->chunk_size + p->N;
    return (int64_t)p->B * ((p->T + p->chunk_size - 1) / p->chunk_size);
}

constexpr int kArrays = 8;
constexpr int64_t kScratchSlots = 512; // at most this many intra workgroups run at once

size_t scratch_slots(const cdr_problem* p) {
    const int64_t nch = num_slots(p) * value_heads(p);
    return (size_t)(nch < kScratchSlots ? nch : kScratchSlots);
}

struct Layout {
    size_t off[kArrays];
    size_t total;
};

Layout layout(const cdr_problem* p) {
    const size_t nch = (size_t)num_slots(p) * (size_t)value_heads(p), nsc = scratch_slots(p);
    const size_t C = (size_t)p->chunk_size, K = (size_t)p->K, V = (size_t)p->V;
    const size_t bytes[kArrays] = {
        nch * K * K * 4,  // Pn (high and low bf16 parts)
        nch * K * V * 4,  // Bm
        nch * C * K * 2,  // Qp
        nch * C * V * 2,  // Up
        nch * K * 4,      // gC
        nch * V * K * 2,  // Sc
        nsc * K * C * 2 + nsc * 1024 * 4,  // kgT, then the pad area of each slot (intra kernel)
        p->varlen ? (size_t)p->N * 4 : 0,  // chain order of packed sequences (longest first)
    };
    Layout L;
    size_t at = 0;
    for (int i = 0; i < kArrays; ++i) {
        L.off[i] = at;
        at += align_up(bytes[i]);
    }
    L.total = at;
    return L;
}

struct BwdLayout {
    size_t m, gcr, rq, rk, bet, wide, dqp, dkp, total;
};

// backward workspace: NMAT fp32 128 x 128 matrices, four 128-vectors and a word of tile flags per
// (chunk slot, value head), and per-value-head dq, dk partials when value heads are grouped
BwdLayout bwd_layout(const cdr_problem* p) {
    const size_t nch = (size_t)num_slots(p) * (size_t)value_heads(p);
    const size_t tokens = (size_t)p->B * p->T;
    BwdLayout L;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t o = at;
        at += align_up(bytes);
        return o;
    };
    L.m = take(nch * cdr::bwd_matrices() * 128 * 128 * sizeof(float));
    L.gcr = take(nch * 128 * sizeof(float));
    L.rq = take(nch * 128 * sizeof(float));
    L.rk = take(nch * 128 * sizeof(float));
    L.bet = take(nch * 128 * sizeof(float));
    L.wide = take(nch * sizeof(uint32_t));
    const bool grouped = value_heads(p) != p->H;
    L.dqp = take(grouped ? tokens * value_heads(p) * p->K * sizeof(float) : 0);
    L.dkp = take(grouped ? tokens * value_heads(p) * p->K * sizeof(float) : 0);
    L.total = at;
    return L;
}

}  // namespace

extern "C" {

cdr_status cdr_check(const cdr_problem* p) {
    if (p == nullptr) return CDR_ERR_NULL_ARG;
    if (p->B <= 0 || p->T < 0 || p->H <= 0 || p->N <= 0 || p->K <= 0 || p->V <= 0 || p->HV < 0)
        return CDR_ERR_BAD_SHAPE;
    if (value_heads(p) % p->H != 0) return CDR_ERR_BAD_SHAPE;  // whole groups of value heads per key head
    if (p->K != 128 || p->V != 128) return CDR_ERR_UNSUPPORTED;
    if (p->chunk_size != 64 && p->chunk_size != 128) return CDR_ERR_UNSUPPORTED;
    if (p->gate != CDR_GATE_PER_DIM && p->gate != CDR_GATE_PER_HEAD) return CDR_ERR_UNSUPPORTED;
    if (p->varlen) {
        if (p->B != 1) return CDR_ERR_VARLEN_BATCH;
    } else if (p->N != p->B) {
        return CDR_ERR_BAD_SHAPE;
    }
    // packed token offsets are int32 on the device side of the interface
    if ((int64_t)p->B * p->T > INT32_MAX) return CDR_ERR_BAD_SHAPE;
    if (num_slots(p) * value_heads(p) > (int64_t)INT32_MAX) return CDR_ERR_BAD_SHAPE;
    return CDR_OK;
}

size_t cdr_workspace_bytes(const cdr_problem* p) {
    if (cdr_check(p) != CDR_OK) return 0;
    return layout(p).total;
}

cdr_status chunk_dr_fwd_stages(const cdr_problem* p, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const float* initial_state,
                               const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
                               size_t workspace_bytes, int32_t stages, void* stream) {
    const cdr_status st = cdr_check(p);
    if (stages < 1 || stages > CDR_STAGE_ALL) return CDR_ERR_UNSUPPORTED;
    if (st != CDR_OK) return st;
    const int64_t tokens = (int64_t)p->B * p->T;
    if (tokens > 0 && (!q || !k || !v || !g || !beta || ((stages & CDR_STAGE_OUTPUT) && !o))) return CDR_ERR_NULL_ARG;
    if (p->has_initial_state && !initial_state) return CDR_ERR_NULL_ARG;
    if (p->output_final_state && !final_state) return CDR_ERR_NULL_ARG;
    if (p->varlen && !cu_seqlens) return CDR_ERR_NULL_ARG;
    const Layout L = layout(p);
    if (workspace == nullptr || workspace_bytes < L.total) return CDR_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return CDR_ERR_WORKSPACE;

    char* wb = static_cast<char*>(workspace);
    cdr::Work ws;
    ws.Pn = reinterpret_cast<uint16_t*>(wb + L.off[0]);
    ws.Bm = reinterpret_cast<float*>(wb + L.off[1]);
    ws.Qp = reinterpret_cast<uint16_t*>(wb + L.off[2]);
    ws.Up = reinterpret_cast<uint16_t*>(wb + L.off[3]);
    ws.gC = reinterpret_cast<float*>(wb + L.off[4]);
    ws.Sc = reinterpret_cast<uint16_t*>(wb + L.off[5]);
    ws.kgT = reinterpret_cast<uint16_t*>(wb + L.off[6]);

    cdr::ChunkMap map;
    map.cu = p->varlen ? cu_seqlens : nullptr;
    map.T = p->T;
    map.N = p->N;
    map.C = p->chunk_size;
    map.nchunk = (p->T + p->chunk_size - 1) / p->chunk_size;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int nslots = (int)num_slots(p);
    const float* s0 = p->has_initial_state ? initial_state : nullptr;
    float* s_out = p->output_final_state ? final_state : nullptr;
    const int C = p->chunk_size;

    if ((stages & CDR_STAGE_INTRA) && nslots > 0) {
        if (cdr::launch_intra(C, p->gate == CDR_GATE_PER_DIM, static_cast<const uint16_t*>(q),
                              static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), g, beta, map,
                              nslots, (int)value_heads(p), p->H, p->qk_l2norm != 0, p->scale, ws,
                              (int)scratch_slots(p), s) != hipSuccess)
            return CDR_ERR_HIP;
    }
    int32_t* order_ws = p->varlen ? reinterpret_cast<int32_t*>(wb + L.off[7]) : nullptr;
    if (stages & CDR_STAGE_CHAIN) {
        if (cdr::launch_chain(map, p->N, (int)value_heads(p), s0, s_out, ws, order_ws, s) != hipSuccess)
            return CDR_ERR_HIP;
    }
    if ((stages & CDR_STAGE_OUTPUT) && nslots > 0) {
        if (cdr::launch_output(C, map, nslots, (int)value_heads(p), static_cast<uint16_t*>(o), ws, s) != hipSuccess)
            return CDR_ERR_HIP;
    }
    return CDR_OK;
}

cdr_status chunk_dr_fwd(const cdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* initial_state, const int32_t* cu_seqlens, void* o,
                        float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_dr_fwd_stages(p, q, k, v, g, beta, initial_state, cu_seqlens, o, final_state, workspace,
                               workspace_bytes, CDR_STAGE_ALL, stream);
}

namespace {

constexpr int kCuCheckThreads = 256;

// One workgroup: every offset is checked against its rules, the smallest failing index + 1 is
// reduced in LDS, and thread 0 writes it (0 when none fails).  The result is written on every
// call, so nothing needs clearing beforehand.
__global__ __launch_bounds__(kCuCheckThreads) void cu_check_kernel(const int32_t* __restrict__ cu, int32_t N, int32_t T,
                                                                   int32_t* __restrict__ result) {
    __shared__ int32_t first;
    if (threadIdx.x == 0) first = N + 2;
    __syncthreads();
    int32_t mine = N + 2;
    for (int32_t i = (int32_t)threadIdx.x; i <= N; i += kCuCheckThreads) {
        const int32_t c = cu[i];
        const bool bad = (c < 0) || (c > T) || (i == 0 && c != 0) || (i > 0 && c < cu[i - 1]) || (i == N && c != T);
        if (bad) {
            mine = i + 1;
            break;  // i grows, so this is the thread's first failure
        }
    }
    if (mine <= N + 1) atomicMin(&first, mine);
    __syncthreads();
    if (threadIdx.x == 0) *result = first <= N + 1 ? first : 0;
}

}  // namespace

cdr_status cdr_check_cu_seqlens(const int32_t* cu_seqlens, int32_t N, int32_t T, int32_t* result, void* stream) {
    if (!cu_seqlens || !result) return CDR_ERR_NULL_ARG;
    if (N < 1 || T < 0) return CDR_ERR_BAD_SHAPE;
    hipLaunchKernelGGL(cu_check_kernel, dim3(1), dim3(kCuCheckThreads), 0, static_cast<hipStream_t>(stream),
                       cu_seqlens, N, T, result);
    return hipGetLastError() == hipSuccess ? CDR_OK : CDR_ERR_HIP;
}

cdr_status chunk_dr_segment_map(const cdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const int32_t* cu_seqlens, float* M, float* X, void* workspace,
                                size_t workspace_bytes, void* stream) {
    const cdr_status st = cdr_check(p);
    if (st != CDR_OK) return st;
    if (!M || !X) return CDR_ERR_NULL_ARG;
    // the offsets X: the forward's final state from a zero start (no output written)
    cdr_problem pz = *p;
    pz.has_initial_state = 0;
    pz.output_final_state = 1;
    const cdr_status s1 = chunk_dr_fwd_stages(&pz, q, k, v, g, beta, nullptr, cu_seqlens, nullptr, X, workspace,
                                              workspace_bytes, CDR_STAGE_INTRA | CDR_STAGE_CHAIN, stream);
    if (s1 != CDR_OK) return s1;
    // the linear part M: the same chunk maps, from the identity and without their offsets
    const Layout L = layout(p);
    char* wb = static_cast<char*>(workspace);
    cdr::Work ws;
    ws.Pn = reinterpret_cast<uint16_t*>(wb + L.off[0]);
    ws.Bm = reinterpret_cast<float*>(wb + L.off[1]);
    ws.gC = reinterpret_cast<float*>(wb + L.off[4]);
    ws.Sc = reinterpret_cast<uint16_t*>(wb + L.off[5]);
    cdr::ChunkMap map;
    map.cu = p->varlen ? cu_seqlens : nullptr;
    map.T = p->T;
    map.N = p->N;
    map.C = p->chunk_size;
    map.nchunk = (p->T + p->chunk_size - 1) / p->chunk_size;
    int32_t* order_ws = p->varlen ? reinterpret_cast<int32_t*>(wb + L.off[7]) : nullptr;
    if (cdr::launch_chain_map(map, p->N, (int)value_heads(p), M, ws, order_ws, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return CDR_ERR_HIP;
    return CDR_OK;
}

cdr_status chunk_dr_merge_states(int32_t R, int32_t HV, int32_t K, int32_t V, const float* M, const float* X,
                                 const float* initial_state, float* s_in, void* stream) {
    if (R <= 0 || HV <= 0 || K <= 0 || V <= 0) return CDR_ERR_BAD_SHAPE;
    if (K != 128 || V != 128) return CDR_ERR_UNSUPPORTED;
    if (!M || !X || !s_in) return CDR_ERR_NULL_ARG;
    return cdr::launch_merge(R, HV, M, X, initial_state, s_in, static_cast<hipStream_t>(stream)) == hipSuccess
               ? CDR_OK
               : CDR_ERR_HIP;
}

size_t cdr_bwd_workspace_bytes(const cdr_problem* p) {
    if (cdr_check(p) != CDR_OK) return 0;
    return bwd_layout(p).total;
}

cdr_status chunk_dr_bwd_stages(const cdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                               const void* d_o, const float* dht, float* dq, float* dk, float* dv, float* dg,
                               float* dbeta, float* dh0, void* workspace, size_t workspace_bytes, int32_t stages,
                               void* stream) {
    const cdr_status st = cdr_check(p);
    if (stages < 1 || stages > CDR_BWD_ALL) return CDR_ERR_UNSUPPORTED;
    if (st != CDR_OK) return st;
    const int64_t tokens = (int64_t)p->B * p->T;
    if (tokens > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
        return CDR_ERR_NULL_ARG;
    if (p->has_initial_state && (!initial_state || !dh0)) return CDR_ERR_NULL_ARG;
    if (p->varlen && !cu_seqlens) return CDR_ERR_NULL_ARG;
    const BwdLayout L = bwd_layout(p);
    if (workspace == nullptr || workspace_bytes < L.total) return CDR_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return CDR_ERR_WORKSPACE;
    const int nslots = tokens > 0 ? (int)num_slots(p) : 0;
    char* wb = static_cast<char*>(workspace);
    cdr::bwd::Work w;
    w.M = reinterpret_cast<float*>(wb + L.m);
    w.gcr = reinterpret_cast<float*>(wb + L.gcr);
    w.rq = reinterpret_cast<float*>(wb + L.rq);
    w.rk = reinterpret_cast<float*>(wb + L.rk);
    w.bet = reinterpret_cast<float*>(wb + L.bet);
    w.wide = reinterpret_cast<uint32_t*>(wb + L.wide);
    const bool grouped = value_heads(p) != p->H;
    w.dqp = grouped ? reinterpret_cast<float*>(wb + L.dqp) : nullptr;
    w.dkp = grouped ? reinterpret_cast<float*>(wb + L.dkp) : nullptr;
    cdr::bwd::In in;
    in.q = static_cast<const uint16_t*>(q);
    in.k = static_cast<const uint16_t*>(k);
    in.v = static_cast<const uint16_t*>(v);
    in.g = g;
    in.beta = beta;
    in.dO = static_cast<const uint16_t*>(d_o);
    in.dq = dq;
    in.dk = dk;
    in.dv = dv;
    in.dg = dg;
    in.dbeta = dbeta;
    cdr::ChunkMap map;
    map.cu = p->varlen ? cu_seqlens : nullptr;
    map.T = p->T;
    map.N = p->N;
    map.C = p->chunk_size;
    map.nchunk = (p->T + p->chunk_size - 1) / p->chunk_size;
    const hipError_t e = cdr::bwd::launch(p->chunk_size, p->gate == CDR_GATE_PER_DIM, p->qk_l2norm != 0, in, map,
                                          nslots, p->N, (int)value_heads(p), p->H, p->scale,
                                          p->has_initial_state ? initial_state : nullptr, dht,
                                          p->has_initial_state ? dh0 : nullptr, w, tokens, stages,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CDR_OK : CDR_ERR_HIP;
}

cdr_status chunk_dr_bwd(const cdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* initial_state, const int32_t* cu_seqlens, const void* d_o,
                        const float* dht, float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_dr_bwd_stages(p, q, k, v, g, beta, initial_state, cu_seqlens, d_o, dht, dq, dk, dv, dg, dbeta, dh0,
                               workspace, workspace_bytes, CDR_BWD_ALL, stream);
}

const char* cdr_status_str(cdr_status s) {
    switch (s) {
        case CDR_OK: return "ok";
        case CDR_ERR_NULL_ARG: return "a required pointer is NULL";
        case CDR_ERR_BAD_SHAPE: return "non-positive or inconsistent sizes";
        case CDR_ERR_UNSUPPORTED: return "unsupported configuration (K and V must be 128, chunk_size 64 or 128)";
        case CDR_ERR_VARLEN_BATCH: return "cu_seqlens requires B == 1";
        case CDR_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case CDR_ERR_HIP: return "HIP kernel launch failed";
        case CDR_ERR_SCRATCH_LIMIT: return "problem needs more workspace than the no-allocation entry point's static array";
    }
    return "unknown status";
}

int32_t cdr_version(void) { return CDR_VERSION; }

}  // extern "C"
