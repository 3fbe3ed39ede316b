// Split-K combine: merge per-chunk partials by their log-sum-exp.
//
// Each context chunk p of sequence b left, per query row, the softmax output
// O_p normalised over the chunk's visible rows and lse_p = ln sum exp(score)
// over them (-inf if it saw none).  Softmax over the union of the chunks is
//   lse = ln sum_p exp(lse_p),   o = sum_p exp(lse_p - lse) O_p,
// which is what this kernel writes (o = 0, lse = -inf when every lse_p is
// -inf).  The up-projection W_UV of the absorb path is linear and was already
// applied per chunk, so the same merge serves both decode paths.
//
// One wave per query row (b, s, h); lanes stride the d_h outputs.  Chunks of
// sequence b are those with p * chunk < L_b (the others were never written), or all
// n_all chunks when n_all > 0 (the sparse path, whose chunks split an index list).
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

// Loads are issued NB partials at a time with clamped, unconditional addresses (entries
// past the last partial get weight 0), so a row's loads overlap instead of waiting for
// one another.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, const int32_t* __restrict__ ctx_lens,
    int max_ctx, int chunk, int n_all, int batch, int s_q, int h_q, int d_h, void* __restrict__ out,
    float* __restrict__ lse_out) {
    constexpr int NB = 4;
    const int rows = batch * s_q * h_q;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int b = row / (s_q * h_q);
    const int nvalid = n_all > 0 ? n_all : (clampi(ctx_lens[b], 0, max_ctx) + chunk - 1) / chunk;
    const size_t plane = (size_t)rows;   // rows per chunk plane
    const int dl = d_h - 1;

    float m = kNegInf;
    for (int p0 = 0; p0 < nvalid; p0 += NB) {
        float lp[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) lp[k] = part_lse[(size_t)min(p0 + k, nvalid - 1) * plane + row];
#pragma unroll
        for (int k = 0; k < NB; ++k) m = fmaxf(m, lp[k]);
    }
    float z = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};   // d_h <= 256: lane handles d = lane + 64k
    if (m != kNegInf) {
        for (int p0 = 0; p0 < nvalid; p0 += NB) {
            float lp[NB], po[NB][4];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const size_t pr = (size_t)min(p0 + k, nvalid - 1) * plane + row;
                lp[k] = part_lse[pr];
#pragma unroll
                for (int q = 0; q < 4; ++q) po[k][q] = part_o[pr * d_h + min(lane + 64 * q, dl)];
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const float w = (p0 + k < nvalid && lp[k] != kNegInf) ? __expf(lp[k] - m) : 0.f;
                z += w;
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] += w * po[k][q];
            }
        }
    }
    const float inv = z > 0.f ? 1.f / z : 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int d = lane + 64 * k;
        if (d < d_h) {
            const float v = acc[k] * inv;
            if (BF16) {
                static_cast<u16*>(out)[(size_t)row * d_h + d] = f2bf(v);
            } else {
                static_cast<float*>(out)[(size_t)row * d_h + d] = v;
            }
        }
    }
    if (lse_out && lane == 0) lse_out[row] = z > 0.f ? m + __logf(z) : kNegInf;
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, bool out_bf16, hipStream_t st) {
    const int rows = a.batch * a.s_q * a.h_q;
    if (rows == 0) return hipSuccess;
    dim3 grid((rows + 3) / 4);
    if (out_bf16) {
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, st, a.part_o, a.part_lse, a.ctx_lens, a.max_ctx,
                           a.chunk, a.n_merge, a.batch, a.s_q, a.h_q, a.d_h, a.out, a.lse);
    } else {
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, st, a.part_o, a.part_lse, a.ctx_lens,
                           a.max_ctx, a.chunk, a.n_merge, a.batch, a.s_q, a.h_q, a.d_h, a.out, a.lse);
    }
    return hipGetLastError();
}

}  // namespace gqla
