// fp32 vector-ALU kernels (generic small dims): expansion, absorb and GQA decode.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Architecture).  Same arithmetic as
// the bf16 MFMA kernels, written for fp32 storage and shapes that are not
// multiples of the MFMA tiles (the decode launchers below take the fp32 MFMA
// kernels of f32_mfma.hip whenever the shape fits them): one workgroup per
// (context chunk, sequence, query row), scores of the chunk in LDS, two-pass
// softmax within the chunk, and the chunk's normalised output plus log-sum-exp
// as the split-K partial.
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

constexpr int NT = 256;
constexpr int kMaxRk = 1024, kMaxDr = 256, kMaxDh = 256;

__device__ float block_reduce_max(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, red[w]);
    return r;
}

__device__ float block_reduce_sum(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < NT / 64; ++w) r += red[w];
    return r;
}

// Softmax over sc[0..n) in place (log2-domain scores, -inf = masked); returns
// (max, sum) through m / l.  Must be called by the whole block.
__device__ void chunk_softmax(float* sc, int n, float* red, float& m, float& l) {
    float mx = kNegInf;
    for (int t = threadIdx.x; t < n; t += NT) mx = fmaxf(mx, sc[t]);
    m = block_reduce_max(mx, red);
    const float muse = m == kNegInf ? 0.f : m;
    float sum = 0.f;
    for (int t = threadIdx.x; t < n; t += NT) {
        const float pv = exp2f(sc[t] - muse);
        sc[t] = pv;
        sum += pv;
    }
    l = block_reduce_sum(sum, red);
}

// grid = (n_split, batch, s_q*h_q); query row rho = s*h_q + h
__global__ __launch_bounds__(NT) void absorb_f32_kernel(
    const float* __restrict__ q_nope, const float* __restrict__ q_rope, const float* __restrict__ w_uk,
    const float* __restrict__ w_uv, const float* __restrict__ cache, int64_t bstride,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int h_q, int g, int s_q, int r_kv, int d_r, int d_h,
    int chunk, int batch, float scale_log2, float* __restrict__ part_o, float* __restrict__ part_lse) {
    __shared__ float qh[kMaxRk + kMaxDr];
    __shared__ float u[kMaxRk];
    __shared__ float sc[kF32MaxChunk];
    __shared__ float red[NT / 64];

    const int p = blockIdx.x, b = blockIdx.y, rho = blockIdx.z;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int t0 = p * chunk;
    if (t0 >= L) return;
    const int s = rho / h_q, h = rho - s * h_q;
    const int j = h / (h_q / g);
    const int nvis = clampi(L - s_q + s + 1, 0, L);
    const int t1 = min(min(t0 + chunk, L), max(nvis, t0));
    const int n = t1 - t0;          // visible rows of this chunk (may be 0)
    const int W = r_kv + d_r;
    const size_t qrow = ((size_t)b * s_q + s) * h_q + h;

    // absorbed query: q~[r] = sum_d W_UK[j][d][r] q^N[d]
    for (int r = threadIdx.x; r < r_kv; r += NT) {
        float acc = 0.f;
        for (int d = 0; d < d_h; ++d) acc += w_uk[((size_t)j * d_h + d) * r_kv + r] * q_nope[qrow * d_h + d];
        qh[r] = acc;
    }
    for (int e = threadIdx.x; e < d_r; e += NT) qh[r_kv + e] = q_rope[qrow * d_r + e];
    __syncthreads();

    const float* seq = cache + (size_t)b * bstride;
    for (int t = threadIdx.x; t < n; t += NT) {
        const float* row = seq + (size_t)(t0 + t) * W;
        float acc = 0.f;
        for (int k = 0; k < W; ++k) acc += qh[k] * row[k];
        sc[t] = acc * scale_log2;
    }
    __syncthreads();
    float m, l;
    chunk_softmax(sc, n, red, m, l);
    __syncthreads();
    const float inv = l > 0.f ? 1.f / l : 0.f;
    for (int r = threadIdx.x; r < r_kv; r += NT) {
        float acc = 0.f;
        for (int t = 0; t < n; ++t) acc += sc[t] * seq[(size_t)(t0 + t) * W + r];
        u[r] = acc * inv;
    }
    __syncthreads();
    const size_t prow = ((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h;
    for (int d = threadIdx.x; d < d_h; d += NT) {
        float acc = 0.f;
        for (int r = 0; r < r_kv; ++r) acc += w_uv[((size_t)j * d_h + d) * r_kv + r] * u[r];
        part_o[prow * d_h + d] = acc;
    }
    if (threadIdx.x == 0) part_lse[prow] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
}

__global__ __launch_bounds__(NT) void gqa_f32_kernel(
    const float* __restrict__ q_nope, const float* __restrict__ q_rope, const float* __restrict__ cache,
    int64_t bstride, const int32_t* __restrict__ ctx_lens, int max_ctx, int h_q, int g, int s_q, int d_r, int d_h,
    int chunk, int batch, float scale_log2, float* __restrict__ part_o, float* __restrict__ part_lse) {
    __shared__ float qv[kMaxDh + kMaxDr];
    __shared__ float sc[kF32MaxChunk];
    __shared__ float red[NT / 64];

    const int p = blockIdx.x, b = blockIdx.y, rho = blockIdx.z;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int t0 = p * chunk;
    if (t0 >= L) return;
    const int s = rho / h_q, h = rho - s * h_q;
    const int j = h / (h_q / g);
    const int nvis = clampi(L - s_q + s + 1, 0, L);
    const int t1 = min(min(t0 + chunk, L), max(nvis, t0));
    const int n = t1 - t0;
    const int W = 2 * g * d_h + d_r;
    const size_t qrow = ((size_t)b * s_q + s) * h_q + h;

    for (int k = threadIdx.x; k < d_h + d_r; k += NT)
        qv[k] = k < d_h ? q_nope[qrow * d_h + k] : q_rope[qrow * d_r + (k - d_h)];
    __syncthreads();

    const float* seq = cache + (size_t)b * bstride;
    for (int t = threadIdx.x; t < n; t += NT) {
        const float* row = seq + (size_t)(t0 + t) * W;
        float acc = 0.f;
        for (int k = 0; k < d_h; ++k) acc += qv[k] * row[j * d_h + k];
        for (int e = 0; e < d_r; ++e) acc += qv[d_h + e] * row[2 * g * d_h + e];
        sc[t] = acc * scale_log2;
    }
    __syncthreads();
    float m, l;
    chunk_softmax(sc, n, red, m, l);
    __syncthreads();
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t prow = ((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h;
    for (int d = threadIdx.x; d < d_h; d += NT) {
        float acc = 0.f;
        for (int t = 0; t < n; ++t) acc += sc[t] * seq[(size_t)(t0 + t) * W + (g + j) * d_h + d];
        part_o[prow * d_h + d] = acc * inv;
    }
    if (threadIdx.x == 0) part_lse[prow] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
}

// grid = (ceil(tokens / 4), batch); 4 tokens per block, thread per output column
__global__ __launch_bounds__(NT) void expand_f32_kernel(
    const float* __restrict__ latent, int64_t lbs, const float* __restrict__ w_uk, const float* __restrict__ w_uv,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int row_begin, int g, int r_kv, int d_r, int d_h,
    float* __restrict__ gc, int64_t gbs) {
    const int b = blockIdx.y;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int WIN = r_kv + d_r, WOUT = 2 * g * d_h + d_r;
    for (int tt = 0; tt < 4; ++tt) {
        const int t = row_begin + blockIdx.x * 4 + tt;
        if (t >= L) return;
        const float* c = latent + (size_t)b * lbs + (size_t)t * WIN;
        float* o = gc + (size_t)b * gbs + (size_t)t * WOUT;
        for (int col = threadIdx.x; col < WOUT; col += NT) {
            if (col < 2 * g * d_h) {
                const float* w = col < g * d_h ? w_uk + (size_t)col * r_kv : w_uv + (size_t)(col - g * d_h) * r_kv;
                float acc = 0.f;
                for (int r = 0; r < r_kv; ++r) acc += w[r] * c[r];
                o[col] = acc;
            } else {
                o[col] = c[r_kv + (col - 2 * g * d_h)];
            }
        }
    }
}

}  // namespace

hipError_t launch_absorb_f32(const DecodeArgs& a, hipStream_t st) {
    if (absorb_f32_mfma_fits(a)) return launch_absorb_f32_mfma(a, st);
    dim3 grid(a.n_split, a.batch, a.s_q * a.h_q);
    hipError_t e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(absorb_f32_kernel, grid, dim3(NT), 0, st, (const float*)a.q_nope, (const float*)a.q_rope,
                       (const float*)a.w_uk, (const float*)a.w_uv, (const float*)a.cache, a.bstride, a.ctx_lens,
                       a.max_ctx, a.h_q, a.g, a.s_q, a.r_kv, a.d_r, a.d_h, a.chunk, a.batch, a.scale * kLog2e,
                       a.part_o, a.part_lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

hipError_t launch_gqa_f32(const DecodeArgs& a, hipStream_t st) {
    if (gqa_f32_mfma_fits(a)) return launch_gqa_f32_mfma(a, st);
    dim3 grid(a.n_split, a.batch, a.s_q * a.h_q);
    hipError_t e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gqa_f32_kernel, grid, dim3(NT), 0, st, (const float*)a.q_nope, (const float*)a.q_rope,
                       (const float*)a.cache, a.bstride, a.ctx_lens, a.max_ctx, a.h_q, a.g, a.s_q, a.d_r, a.d_h,
                       a.chunk, a.batch, a.scale * kLog2e, a.part_o, a.part_lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

hipError_t launch_expand_f32(const ExpandArgs& a, hipStream_t st) {
    const int span = a.max_ctx - a.row_begin;
    if (span <= 0 || a.batch == 0) return hipSuccess;
    dim3 grid((span + 3) / 4, a.batch);
    hipLaunchKernelGGL(expand_f32_kernel, grid, dim3(NT), 0, st, (const float*)a.latent, a.latent_bstride,
                       (const float*)a.w_uk, (const float*)a.w_uv, a.ctx_lens, a.max_ctx, a.row_begin, a.g,
                       a.r_kv, a.d_r, a.d_h, (float*)a.group_cache, a.group_bstride);
    return hipGetLastError();
}

}  // namespace gqla
