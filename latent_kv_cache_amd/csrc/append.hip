// Decode-step append: the s_q new tokens of every sequence enter the caches.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Architecture).  Each cached token keeps
// its latent row cKV and one rotary key k_R shared by all heads; each query head has
// its own rotary part q^R.  The decode kernels take keys and queries with the rotary
// embedding already applied, so this step rotates them: new token s of a sequence of
// length L (the new tokens included) sits at position t = L - s_q + s, and
//   latent[b][t]            = [c_new | RoPE_t(k_R)]
//   q_rope_out[b][s][h]     = RoPE_t(q^R_raw[b][s][h])
//   group_cache[b][t]       = [W_UK[0] c .. W_UK[g-1] c | W_UV[0] c .. W_UV[g-1] c | RoPE_t(k_R)]
// the last being the once-per-token expansion of the GQA path, done for the new
// rows only.  RoPE pairs component k with k + d_R/2 and turns the pair by
// t * theta^(-2k/d_R).
//
// The rotation angles, their sines and cosines and the rotated values are computed in
// fp64 and rounded once to fp32 (then, for bf16 storage, from fp32 to bf16, both round
// to nearest even), without fused multiply-adds: positions reach 10^5 and more, where
// an fp32 angle would be off by far more than the storage precision.
#include "common.h"
#include "launch.h"
#include "append_rope.h"

namespace gqla {

namespace {

// grid = batch * s_q blocks (one per new token), 256 threads
template <typename T>
__global__ __launch_bounds__(256) void append_rope_kernel(
    const T* __restrict__ c_new, const T* __restrict__ kr_new, const T* __restrict__ q_raw, T* __restrict__ q_out,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int s_q, int h_q, int r_kv, int d_r, double theta,
    T* __restrict__ latent, int64_t lbs, T* __restrict__ group, int64_t gbs, int gw) {
    append_rope_token<T, 256>(blockIdx.x, c_new, kr_new, q_raw, q_out, ctx_lens, max_ctx, s_q, h_q, r_kv, d_r, theta,
                              latent, lbs, group, gbs, gw);
}

// fp32 expansion of the new rows: grid = batch * s_q blocks, thread per output column
__global__ __launch_bounds__(256) void append_expand_f32_kernel(
    const float* __restrict__ c_new, const float* __restrict__ w_uk, const float* __restrict__ w_uv,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int s_q, int g, int r_kv, int d_h,
    float* __restrict__ group, int64_t gbs, int d_r) {
    const int b = blockIdx.x / s_q, s = blockIdx.x - (blockIdx.x / s_q) * s_q;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int t = L - s_q + s;
    if (t < 0) return;
    const float* c = c_new + ((size_t)b * s_q + s) * r_kv;
    float* o = group + (size_t)b * gbs + (size_t)t * (2 * g * d_h + d_r);
    for (int col = threadIdx.x; col < 2 * g * d_h; col += 256) {
        const float* w = col < g * d_h ? w_uk + (size_t)col * r_kv : w_uv + (size_t)(col - g * d_h) * r_kv;
        float acc = 0.f;
        for (int r = 0; r < r_kv; ++r) acc += w[r] * c[r];
        o[col] = acc;
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, bool bf16, hipStream_t st) {
    const int tokens = a.batch * a.s_q;
    if (tokens == 0) return hipSuccess;
    const int gw = 2 * a.g * a.d_h;
    // bf16 with the group cache: one launch for the rotations and the expansion
    if (bf16 && a.group_cache) return launch_append_fused_bf16(a, st);
    if (bf16) {
        hipLaunchKernelGGL(append_rope_kernel<u16>, dim3(tokens), dim3(256), 0, st, (const u16*)a.c_new,
                           (const u16*)a.kr_new, (const u16*)a.q_rope_raw, (u16*)a.q_rope_out, a.ctx_lens, a.max_ctx,
                           a.s_q, a.h_q, a.r_kv, a.d_r, (double)a.theta, (u16*)a.latent, a.latent_bstride,
                           (u16*)a.group_cache, a.group_bstride, gw);
    } else {
        hipLaunchKernelGGL(append_rope_kernel<float>, dim3(tokens), dim3(256), 0, st, (const float*)a.c_new,
                           (const float*)a.kr_new, (const float*)a.q_rope_raw, (float*)a.q_rope_out, a.ctx_lens,
                           a.max_ctx, a.s_q, a.h_q, a.r_kv, a.d_r, (double)a.theta, (float*)a.latent,
                           a.latent_bstride, (float*)a.group_cache, a.group_bstride, gw);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.group_cache) return e;
    hipLaunchKernelGGL(append_expand_f32_kernel, dim3(tokens), dim3(256), 0, st, (const float*)a.c_new,
                       (const float*)a.w_uk, (const float*)a.w_uv, a.ctx_lens, a.max_ctx, a.s_q, a.g, a.r_kv, a.d_h,
                       (float*)a.group_cache, a.group_bstride, a.d_r);
    return hipGetLastError();
}

}  // namespace gqla
