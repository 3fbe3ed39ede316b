// Rotary part of the decode-step append (see append.hip), as a device function that
// the append's own kernel and the fused bf16 append kernel (expand_bf16.hip) share.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Architecture): one latent row and one shared
// rotary key per cached token, a rotary query part per head.
#pragma once
#include "common.h"

namespace gqla {

namespace {

__device__ __forceinline__ double to_f64(u16 v) { return (double)bf2f(v); }
__device__ __forceinline__ double to_f64(float v) { return (double)v; }
__device__ __forceinline__ void store_from_f64(u16* p, double x) { *p = f2bf((float)x); }
__device__ __forceinline__ void store_from_f64(float* p, double x) { *p = (float)x; }

constexpr int kMaxHalf = 128;   // d_R <= 256

// New token `token` (= b * s_q + s) of the append, by one block of NT threads: its latent
// row, its rotated key (in the latent row and, with group, in the group row) and its
// heads' rotated queries.
template <typename T, int NT>
__device__ __forceinline__ void append_rope_token(
    int token, const T* __restrict__ c_new, const T* __restrict__ kr_new, const T* __restrict__ q_raw,
    T* __restrict__ q_out, const int32_t* __restrict__ ctx_lens, int max_ctx, int s_q, int h_q, int r_kv, int d_r,
    double theta, T* __restrict__ latent, int64_t lbs, T* __restrict__ group, int64_t gbs, int gw) {
#pragma clang fp contract(off)
    __shared__ double cs[kMaxHalf], sn[kMaxHalf];
    const int b = token / s_q, s = token - (token / s_q) * s_q;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int t = L - s_q + s;
    if (t < 0) return;   // the sequence is shorter than its new tokens: no row for this one
    const int half = d_r / 2;
    const int tid = threadIdx.x;
    for (int k = tid; k < half; k += NT) {
        const double f = pow(theta, (-2.0 * (double)k) / (double)d_r);
        const double a = (double)t * f;
        cs[k] = cos(a);
        sn[k] = sin(a);
    }
    __syncthreads();

    const size_t tok = (size_t)b * s_q + s;
    T* row = latent + (size_t)b * lbs + (size_t)t * (r_kv + d_r);
    const T* cn = c_new + tok * r_kv;
    for (int e = tid; e < r_kv; e += NT) row[e] = cn[e];

    const T* kr = kr_new + tok * d_r;
    T* grow = group ? group + (size_t)b * gbs + (size_t)t * (gw + d_r) + gw : nullptr;
    for (int k = tid; k < half; k += NT) {
        const double x = to_f64(kr[k]), y = to_f64(kr[k + half]);
        const double r0 = x * cs[k] - y * sn[k];
        const double r1 = x * sn[k] + y * cs[k];
        store_from_f64(row + r_kv + k, r0);
        store_from_f64(row + r_kv + k + half, r1);
        if (grow) {
            store_from_f64(grow + k, r0);
            store_from_f64(grow + k + half, r1);
        }
    }
    if (q_raw) {
        const T* qs = q_raw + tok * h_q * d_r;
        T* qd = q_out + tok * h_q * d_r;
        for (int i = tid; i < h_q * half; i += NT) {
            const int h = i / half, k = i - (i / half) * half;
            const double x = to_f64(qs[h * d_r + k]), y = to_f64(qs[h * d_r + k + half]);
            store_from_f64(qd + h * d_r + k, x * cs[k] - y * sn[k]);
            store_from_f64(qd + h * d_r + k + half, x * sn[k] + y * cs[k]);
        }
    }
}


}  // namespace

}  // namespace gqla
