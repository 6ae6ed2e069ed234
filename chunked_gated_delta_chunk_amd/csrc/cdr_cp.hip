// Merge of per-segment state maps (the exchange step of context parallelism, page
// "flash-linear-attention KCP 精度失效根因排查手册", the merge that turns each rank's segment
// summary into the state that really enters the next segment).
//
// A segment run from a zero state ends in X, and its final state from any start S is
// S M + X (both [V, K], M [K, K], the state's rows evolving independently).  Given the
// segments in order, s_in[0] = s0 and s_in[r + 1] = s_in[r] M[r] + X[r].  Rows of the state
// are independent, so a workgroup owns 16 rows of one value head for all segments; M[r] is
// staged in LDS one segment at a time.
#include "cdr_common.h"

namespace cdr {

namespace {

constexpr int MROWS = 16;                 // state rows per workgroup
constexpr int MTHREADS = 512;             // 32 threads per row, four columns each

__global__ __launch_bounds__(MTHREADS) void merge_kernel(int R, int HV, const float* __restrict__ M,
                                                         const float* __restrict__ X, const float* __restrict__ s0,
                                                         float* __restrict__ s_in) {
    __shared__ __attribute__((aligned(16))) float sM[KD * KD];
    __shared__ __attribute__((aligned(16))) float sS[MROWS * KD];
    const int hv = blockIdx.x, rb = blockIdx.y;
    const int tid = threadIdx.x, r = tid >> 5, c0 = 4 * (tid & 31);
    const int v = MROWS * rb + r;
    const size_t st = (size_t)VD * KD;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (s0 != nullptr) s = *reinterpret_cast<const float4*>(s0 + (size_t)hv * st + (size_t)v * KD + c0);
    *reinterpret_cast<float4*>(s_in + (size_t)hv * st + (size_t)v * KD + c0) = s;
    for (int seg = 0; seg < R; ++seg) {
        const float* Mr = M + ((size_t)seg * HV + hv) * KD * KD;
        __syncthreads();  // the previous segment's operands are no longer read
        for (int e = tid; e < KD * KD / 4; e += MTHREADS)
            *reinterpret_cast<float4*>(sM + 4 * e) = *reinterpret_cast<const float4*>(Mr + 4 * e);
        *reinterpret_cast<float4*>(sS + r * KD + c0) = s;
        __syncthreads();
        float4 acc = *reinterpret_cast<const float4*>(X + ((size_t)seg * HV + hv) * st + (size_t)v * KD + c0);
#pragma unroll 8
        for (int a = 0; a < KD; ++a) {
            const float sa = sS[r * KD + a];
            const float4 m = *reinterpret_cast<const float4*>(sM + a * KD + c0);
            acc.x += sa * m.x;
            acc.y += sa * m.y;
            acc.z += sa * m.z;
            acc.w += sa * m.w;
        }
        s = acc;
        *reinterpret_cast<float4*>(s_in + ((size_t)(seg + 1) * HV + hv) * st + (size_t)v * KD + c0) = s;
    }
}

}  // namespace

hipError_t launch_merge(int R, int HV, const float* M, const float* X, const float* s0, float* s_in,
                        hipStream_t stream) {
    hipLaunchKernelGGL(merge_kernel, dim3(HV, VD / MROWS), dim3(MTHREADS), 0, stream, R, HV, M, X, s0, s_in);
    return hipGetLastError();
}

}  // namespace cdr
