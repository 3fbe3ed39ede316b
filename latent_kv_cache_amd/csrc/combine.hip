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
// One wave per query row (b, s, h); each lane holds d_h/64 consecutive outputs.  Chunks of
// sequence b are those with p * chunk < L_b (the others were never written), or all
// n_all chunks when n_all > 0 (the sparse path, whose chunks split an index list).
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

// Loads are issued NB partials at a time with clamped, unconditional addresses (entries
// past the last partial get weight 0), so a row's loads overlap instead of waiting for
// one another.  Lane l holds the E = d_h/64 consecutive outputs d = E*l .. E*l + E-1
// (one vector load per partial); with E = 1 and d_h < 64 the upper lanes hold nothing.
template <int E>
__device__ __forceinline__ void load_e(const float* p, float (&v)[E]) {
    if constexpr (E == 4) {
        const floatx4 x = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = x[e];
    } else if constexpr (E == 2) {
        const floatx2 x = *reinterpret_cast<const floatx2*>(p);
        v[0] = x[0];
        v[1] = x[1];
    } else {
        v[0] = *p;
    }
}

template <bool BF16, int E>
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
    const bool mine = E * lane < d_h;    // E * 64 >= d_h, and d_h is a multiple of E
    const int d0 = mine ? E * lane : 0;

    float m = kNegInf;
    float z = 0.f;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    // A partial with lse_p = -inf gets weight 0, so m = -inf (no chunk saw a token)
    // leaves z = 0 and o = 0 without a separate test.
    if (nvalid >= 1 && nvalid <= NB) {
        // every load of the row at once: one round trip to memory (nvalid = 0, an empty
        // sequence, takes the loop below, which loads nothing)
        float lp[NB], po[NB][E];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const size_t pr = (size_t)min(k, nvalid - 1) * plane + row;
            lp[k] = part_lse[pr];
            load_e<E>(part_o + pr * d_h + d0, po[k]);
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) m = fmaxf(m, lp[k]);   // clamped entries repeat the last
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const float w = (k < nvalid && lp[k] != kNegInf) ? __expf(lp[k] - m) : 0.f;
            z += w;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += w * po[k][e];
        }
    } else {
        for (int p0 = 0; p0 < nvalid; p0 += NB) {
            float lp[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) lp[k] = part_lse[(size_t)min(p0 + k, nvalid - 1) * plane + row];
#pragma unroll
            for (int k = 0; k < NB; ++k) m = fmaxf(m, lp[k]);
        }
        for (int p0 = 0; p0 < nvalid; p0 += NB) {
            float lp[NB], po[NB][E];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const size_t pr = (size_t)min(p0 + k, nvalid - 1) * plane + row;
                lp[k] = part_lse[pr];
                load_e<E>(part_o + pr * d_h + d0, po[k]);
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const float w = (p0 + k < nvalid && lp[k] != kNegInf) ? __expf(lp[k] - m) : 0.f;
                z += w;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[e] += w * po[k][e];
            }
        }
    }
    const float inv = z > 0.f ? 1.f / z : 0.f;
    if (mine) {
        if (BF16) {
            u16* o = static_cast<u16*>(out) + (size_t)row * d_h + d0;
            if constexpr (E == 4) {
                *reinterpret_cast<u32x2*>(o) = u32x2{pack2f(acc[0] * inv, acc[1] * inv), pack2f(acc[2] * inv, acc[3] * inv)};
            } else if constexpr (E == 2) {
                *reinterpret_cast<uint32_t*>(o) = pack2f(acc[0] * inv, acc[1] * inv);
            } else {
                *o = f2bf(acc[0] * inv);
            }
        } else {
            float* o = static_cast<float*>(out) + (size_t)row * d_h + d0;
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = acc[e] * inv;
        }
    }
    if (lse_out && lane == 0) lse_out[row] = z > 0.f ? m + __logf(z) : kNegInf;
}

template <bool BF16>
void launch_combine_t(const DecodeArgs& a, dim3 grid, hipStream_t st) {
    if (a.d_h > 128) {
        hipLaunchKernelGGL((combine_kernel<BF16, 4>), grid, dim3(256), 0, st, a.part_o, a.part_lse, a.ctx_lens,
                           a.max_ctx, a.chunk, a.n_merge, a.batch, a.s_q, a.h_q, a.d_h, a.out, a.lse);
    } else if (a.d_h > 64) {
        hipLaunchKernelGGL((combine_kernel<BF16, 2>), grid, dim3(256), 0, st, a.part_o, a.part_lse, a.ctx_lens,
                           a.max_ctx, a.chunk, a.n_merge, a.batch, a.s_q, a.h_q, a.d_h, a.out, a.lse);
    } else {
        hipLaunchKernelGGL((combine_kernel<BF16, 1>), grid, dim3(256), 0, st, a.part_o, a.part_lse, a.ctx_lens,
                           a.max_ctx, a.chunk, a.n_merge, a.batch, a.s_q, a.h_q, a.d_h, a.out, a.lse);
    }
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, bool out_bf16, hipStream_t st) {
    const int rows = a.batch * a.s_q * a.h_q;
    if (rows == 0) return hipSuccess;
    dim3 grid((rows + 3) / 4);
    if (out_bf16) {
        launch_combine_t<true>(a, grid, st);
    } else {
        launch_combine_t<false>(a, grid, st);
    }
    return hipGetLastError();
}

}  // namespace gqla
