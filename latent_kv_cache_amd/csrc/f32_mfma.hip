// fp32 MFMA decode kernels for gfx950 (16x16x4 fp32 MFMA): absorb and GQA paths.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Architecture): the MQA-absorb path
// (absorbed queries W_UK^T q^N against the latent rows, the value sum in latent
// space, then W_UV) and the GQA path (attention over the once-expanded group rows),
// here for fp32 storage and arithmetic.
//
// Work split.  One workgroup per (context chunk, sequence, group j) holds every query
// row of the group (s_q h_q / g rows, up to 64: four waves of one 16-row tile each), so
// each cached row is read once per group, not once per head.  The chunk streams in
// 16-token tiles staged in LDS.  Each wave computes, for its 16 rows,
//   S^T[token][row] = K_tile . Q^T        (A = cache rows from LDS, B = queries)
// and accumulates
//   O^T[feat][row] += V_tile^T . P^T      (A = cache columns from LDS, B = P)
// with the fp32 products exact and fp32 accumulation.  Lane (q, r) of an MFMA result
// holds rows 4q..4q+3 of column r.  The value product's k-step e takes the tokens
// 4q + e of the tile (a permutation of the contraction), so its B operand is the lane's
// own softmax weight number e: P never leaves the registers.  The absorb path keeps u in
// the same layout and contracts it with W_UV the same way (k-step e of latent tile m
// takes u columns 16 m + 4 q + e).
//
// Softmax: online over the tiles, exact rescale of the accumulators whenever a row's
// maximum rises; the chunk's normalised output and its log-sum-exp are the split-K
// partial, merged by launch_combine.
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

constexpr int FT = 16;          // tokens per tile
constexpr int FW = 4;           // waves per workgroup (one 16-row tile each)
constexpr int FMAXT = 16;       // 16-wide tiles of d_h (GQA) or r_kv (absorb) held in registers

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Online softmax of one tile for the lane's four tokens of row r16: s[v] are log2-domain
// scores (-inf: masked).  m: the row's running maximum (identical in its four lanes), l:
// the lane's partial sum.  Returns the factor the row's accumulators take before this
// tile is added; p receives the tile's weights.
__device__ __forceinline__ float softmax4(const float (&s)[4], float& m, float& l, float (&p)[4]) {
    float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mt = wave_max16x4(mt);
    const float mn = fmaxf(m, mt);
    const float alpha = (mn == kNegInf || m == mn) ? 1.f : exp2f(m - mn);   // m = -inf gives 0
    const float muse = mn == kNegInf ? 0.f : mn;
#pragma unroll
    for (int v = 0; v < 4; ++v) p[v] = exp2f(s[v] - muse);
    l = l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m = mn;
    return alpha;
}

// Stage tokens [tb, tb + FT) of a sequence's rows (row pitch W floats) into tile
// (row stride TS): ncol columns taken from up to three column ranges of the row,
// [c0, c0 + n0), [c1, c1 + n1), [c2, c2 + n2), placed side by side.  Tokens at or past
// t1 stage zeros.
__device__ __forceinline__ void stage_tile(float* tile, int TS, const float* __restrict__ seq, int W, int tb, int t1,
                                           int c0, int n0, int c1, int n1, int c2, int n2) {
    const int ncol = n0 + n1 + n2;
    for (int e = threadIdx.x; e < FT * ncol; e += FW * 64) {
        const int r = e / ncol, c = e - r * ncol;
        const int src = c < n0 ? c0 + c : (c < n0 + n1 ? c1 + (c - n0) : c2 + (c - n0 - n1));
        tile[r * TS + c] = tb + r < t1 ? seq[(size_t)(tb + r) * W + src] : 0.f;
    }
}

// grid = (n_split, batch, g).  Dynamic LDS: FT x TS tile + FW x (d_h + d_r) x 16 queries.
__global__ __launch_bounds__(FW * 64) void gqa_f32_mfma_kernel(
    const float* __restrict__ q_nope, const float* __restrict__ q_rope, const float* __restrict__ cache,
    int64_t bstride, const int32_t* __restrict__ ctx_lens, int max_ctx, int h_q, int g, int s_q, int d_r, int d_h,
    int chunk, int batch, float scale_log2, float* __restrict__ part_o, float* __restrict__ part_lse) {
    extern __shared__ float smem[];
    const int p = blockIdx.x, b = blockIdx.y, j = blockIdx.z;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int t0 = p * chunk;
    if (t0 >= L) return;   // no partial: the combine merges only the chunks below L
    const int t1 = min(t0 + chunk, L);
    const int KQ = d_h + d_r;                 // contraction of the scores
    const int TW = 2 * d_h + d_r;             // staged columns: K_j, V_j, k_R
    const int TS = TW + 1;
    float* tile = smem;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    float* qs = smem + FT * TS + wave * KQ * 16;   // this wave's queries, [k][row]

    const int hpg = h_q / g, rows_g = s_q * hpg;
    const int rho = wave * 16 + r16;          // the lane's query row within the group
    const bool active = wave * 16 < rows_g;
    const bool row_ok = rho < rows_g;
    const int s = row_ok ? rho / hpg : 0;
    const int h = j * hpg + (row_ok ? rho - s * hpg : 0);
    const size_t qrow = ((size_t)b * s_q + s) * h_q + h;
    const int nvis = clampi(L - s_q + s + 1, 0, L);
    if (active) {
        for (int e = lane; e < KQ * 16; e += 64) {
            const int k = e >> 4, r = e & 15, rr = wave * 16 + r;
            float v = 0.f;
            if (rr < rows_g) {
                const int ss = rr / hpg;
                const size_t qr = ((size_t)b * s_q + ss) * h_q + j * hpg + (rr - ss * hpg);
                v = k < d_h ? q_nope[qr * d_h + k] : q_rope[qr * d_r + (k - d_h)];
            }
            qs[e] = v;
        }
    }

    const int ndt = d_h / 16;
    floatx4 o[FMAXT];
#pragma unroll
    for (int t = 0; t < FMAXT; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, l = 0.f;
    const float* seq = cache + (size_t)b * bstride;
    const int W = 2 * g * d_h + d_r;
    for (int tb = t0; tb < t1; tb += FT) {
        __syncthreads();   // the previous tile is consumed (and the queries are staged)
        stage_tile(tile, TS, seq, W, tb, t1, j * d_h, d_h, (g + j) * d_h, d_h, 2 * g * d_h, d_r);
        __syncthreads();
        if (!active) continue;
        // scores: k-step ks contracts columns 4 ks .. 4 ks + 3 (q^N, then q^R against k_R)
        floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < KQ / 4; ++ks) {
            const int k = 4 * ks + q4;
            const float a = tile[r16 * TS + (k < d_h ? k : k + d_h)];
            sacc = mfma4(a, qs[ks * 64 + lane], sacc);
        }
        float sc[4], pw[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = tb + 4 * q4 + v;
            sc[v] = (row_ok && t < t1 && t < nvis) ? sacc[v] * scale_log2 : kNegInf;
        }
        const float alpha = softmax4(sc, m, l, pw);
#pragma unroll
        for (int t = 0; t < FMAXT; ++t)
            if (t < ndt) {
                o[t] *= alpha;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[t] = mfma4(tile[(4 * q4 + e) * TS + d_h + 16 * t + r16], pw[e], o[t]);
            }
    }
    if (!active) return;
    const float lt = wave_sum16x4(l);
    if (!row_ok) return;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const size_t prow = (size_t)p * batch * s_q * h_q + qrow;
#pragma unroll
    for (int t = 0; t < FMAXT; ++t)
        if (t < ndt) {
#pragma unroll
            for (int v = 0; v < 4; ++v) part_o[prow * d_h + 16 * t + 4 * q4 + v] = o[t][v] * inv;
        }
    if (q4 == 0) part_lse[prow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
}

// grid = (n_split, batch, g).  Dynamic LDS: FT x TS tile + FW x (r_kv + d_r) x 16 queries.
__global__ __launch_bounds__(FW * 64) void absorb_f32_mfma_kernel(
    const float* __restrict__ q_nope, const float* __restrict__ q_rope, const float* __restrict__ w_uk,
    const float* __restrict__ w_uv, const float* __restrict__ cache, int64_t bstride,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int h_q, int g, int s_q, int r_kv, int d_r, int d_h,
    int chunk, int batch, float scale_log2, float* __restrict__ part_o, float* __restrict__ part_lse) {
    extern __shared__ float smem[];
    const int p = blockIdx.x, b = blockIdx.y, j = blockIdx.z;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int t0 = p * chunk;
    if (t0 >= L) return;
    const int t1 = min(t0 + chunk, L);
    const int W = r_kv + d_r;                 // latent row: c_t, then k_R,t
    const int TS = W + 1;
    float* tile = smem;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    float* qs = smem + FT * TS + wave * W * 16;    // this wave's absorbed queries, [k][row]

    const int hpg = h_q / g, rows_g = s_q * hpg;
    const int rho = wave * 16 + r16;
    const bool active = wave * 16 < rows_g;
    const bool row_ok = rho < rows_g;
    const int s = row_ok ? rho / hpg : 0;
    const int h = j * hpg + (row_ok ? rho - s * hpg : 0);
    const size_t qrow = ((size_t)b * s_q + s) * h_q + h;
    const int nvis = clampi(L - s_q + s + 1, 0, L);
    const int nmt = r_kv / 16;
    if (active) {
        // absorbed query q~^T[r][row] = W_UK[j]^T[r][d] . q^N^T[d][row], latent tile mt at a time
        for (int mt = 0; mt < nmt; ++mt) {
            floatx4 qa = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks < d_h / 4; ++ks) {
                const int d = 4 * ks + q4;
                const float a = w_uk[((size_t)j * d_h + d) * r_kv + 16 * mt + r16];
                const float bq = row_ok ? q_nope[qrow * d_h + d] : 0.f;
                qa = mfma4(a, bq, qa);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) qs[(16 * mt + 4 * q4 + v) * 16 + r16] = qa[v];
        }
        for (int e = lane; e < d_r * 16; e += 64) {
            const int k = e >> 4, r = e & 15, rr = wave * 16 + r;
            float v = 0.f;
            if (rr < rows_g) {
                const int ss = rr / hpg;
                v = q_rope[(((size_t)b * s_q + ss) * h_q + j * hpg + (rr - ss * hpg)) * d_r + k];
            }
            qs[(r_kv + k) * 16 + r] = v;
        }
    }

    floatx4 u[FMAXT];
#pragma unroll
    for (int t = 0; t < FMAXT; ++t) u[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, l = 0.f;
    const float* seq = cache + (size_t)b * bstride;
    for (int tb = t0; tb < t1; tb += FT) {
        __syncthreads();
        stage_tile(tile, TS, seq, W, tb, t1, 0, W, 0, 0, 0, 0);
        __syncthreads();
        if (!active) continue;
        floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < W / 4; ++ks) sacc = mfma4(tile[r16 * TS + 4 * ks + q4], qs[ks * 64 + lane], sacc);
        float sc[4], pw[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = tb + 4 * q4 + v;
            sc[v] = (row_ok && t < t1 && t < nvis) ? sacc[v] * scale_log2 : kNegInf;
        }
        const float alpha = softmax4(sc, m, l, pw);
        // U^T[r][row] += C^T[r][token] . P^T[token][row]
#pragma unroll
        for (int t = 0; t < FMAXT; ++t)
            if (t < nmt) {
                u[t] *= alpha;
#pragma unroll
                for (int e = 0; e < 4; ++e) u[t] = mfma4(tile[(4 * q4 + e) * TS + 16 * t + r16], pw[e], u[t]);
            }
    }
    if (!active) return;
    const float lt = wave_sum16x4(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // O^T[d][row] = W_UV[j][d][r] . U^T[r][row]: k-step (t, e) takes columns 16 t + 4 q + e
    const size_t prow = (size_t)p * batch * s_q * h_q + qrow;
    for (int dt = 0; dt < d_h / 16; ++dt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const float* wrow = w_uv + ((size_t)j * d_h + 16 * dt + r16) * r_kv + 4 * q4;
#pragma unroll
        for (int t = 0; t < FMAXT; ++t)
            if (t < nmt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(wrow[16 * t + e], u[t][e], acc);
            }
        if (row_ok) {
#pragma unroll
            for (int v = 0; v < 4; ++v) part_o[prow * d_h + 16 * dt + 4 * q4 + v] = acc[v] * inv;
        }
    }
    if (row_ok && q4 == 0) part_lse[prow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
}

constexpr size_t kMfmaLds = 64u << 10;   // dynamic LDS the MFMA kernels may take

size_t gqa_lds(const DecodeArgs& a) {
    return ((size_t)FT * (2 * a.d_h + a.d_r + 1) + (size_t)FW * (a.d_h + a.d_r) * 16) * sizeof(float);
}

size_t absorb_lds(const DecodeArgs& a) {
    return ((size_t)FT * (a.r_kv + a.d_r + 1) + (size_t)FW * (a.r_kv + a.d_r) * 16) * sizeof(float);
}

bool common_fits(const DecodeArgs& a) {
    return a.g > 0 && a.h_q % a.g == 0 && a.s_q * (a.h_q / a.g) <= FW * 16 && a.d_h % 16 == 0 &&
           a.d_h <= 16 * FMAXT && a.d_r % 4 == 0;
}

}  // namespace

bool gqa_f32_mfma_fits(const DecodeArgs& a) { return common_fits(a) && gqa_lds(a) <= kMfmaLds; }

bool absorb_f32_mfma_fits(const DecodeArgs& a) {
    return common_fits(a) && a.r_kv % 16 == 0 && a.r_kv <= 16 * FMAXT && absorb_lds(a) <= kMfmaLds;
}

hipError_t launch_gqa_f32_mfma(const DecodeArgs& a, hipStream_t st) {
    dim3 grid(a.n_split, a.batch, a.g);
    hipError_t e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gqa_f32_mfma_kernel, grid, dim3(FW * 64), gqa_lds(a), st, (const float*)a.q_nope,
                       (const float*)a.q_rope, (const float*)a.cache, a.bstride, a.ctx_lens, a.max_ctx, a.h_q, a.g,
                       a.s_q, a.d_r, a.d_h, a.chunk, a.batch, a.scale * kLog2e, a.part_o, a.part_lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

hipError_t launch_absorb_f32_mfma(const DecodeArgs& a, hipStream_t st) {
    dim3 grid(a.n_split, a.batch, a.g);
    hipError_t e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(absorb_f32_mfma_kernel, grid, dim3(FW * 64), absorb_lds(a), st, (const float*)a.q_nope,
                       (const float*)a.q_rope, (const float*)a.w_uk, (const float*)a.w_uv, (const float*)a.cache,
                       a.bstride, a.ctx_lens, a.max_ctx, a.h_q, a.g, a.s_q, a.r_kv, a.d_r, a.d_h, a.chunk, a.batch,
                       a.scale * kLog2e, a.part_o, a.part_lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

}  // namespace gqla
