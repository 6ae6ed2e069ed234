// Host-side entry points of the backward kernels (cdr_bwd.hip), used by the C interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "cdr_common.h"

namespace cdr {
namespace bwd {

struct Work {
    float* M;      // [nch][bwd_matrices()][128 * 128] per (chunk, value head) matrices
    float* gcr;    // [nch][128] gamma_C (raw)
    float* rq;     // [nch][128] L2 scales of q rows (1 when off)
    float* rk;     // [nch][128] L2 scales of k rows
    float* bet;    // [nch][128] beta of the chunk rows (0 on rows past the end)
    uint32_t* wide;  // [nch] bit t set: the gates of row tile t are too wide for a middle-row pivot
    float* dqp;    // [B*T][HV][K] per-value-head dq (grouped heads), or null
    float* dkp;
};

struct In {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    const float* beta;
    const uint16_t* dO;
    float* dq;
    float* dk;
    float* dv;
    float* dg;
    float* dbeta;
};

hipError_t launch(int C, bool per_dim, bool l2n, const In& in, const ChunkMap& map, int nslots, int N, int H, int Hk,
                  float scale, const float* h0, const float* dht, float* dh0, const Work& w, int64_t tokens,
                  int stages, hipStream_t s);

}  // namespace bwd

int bwd_matrices();  // fp32 128 x 128 matrices per (chunk, value head) in the backward workspace

}  // namespace cdr
