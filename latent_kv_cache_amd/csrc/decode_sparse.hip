// Sparse GQLA decode: GQA attention over per-(query token, group) lists of selected rows.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Sparse GQLA).  Fine-grained sparse
// attention keeps the GQA path because the h_q/g = 16 heads of a group fill one
// 16-row matrix tile: the heads of group j share the selection of query token s,
//   score_t = scale [q^N | q^R].[K_j,t | k_R,t]   for t in indices[b][s][j][:],
//   o = softmax-weighted sum of V_j,t over the listed rows,
// skipping entries outside [0, L_b) or past the token's causal window
// t <= L_b - s_q + s; a row listed twice counts twice.  The index list is split into
// chunks (split-K); each work item writes its chunk's normalised output and
// log-sum-exp and launch_combine merges every chunk.
//
// bf16 kernel.  One wave per work item (sequence, query token, group, 16-row tile of
// the group's heads, list chunk); the four waves of a block are independent, each with
// its own LDS slice, so the kernel has no block barrier.  Per tile of 32 listed rows:
//   - the 32 K_j rows are gathered four rows of 256 bytes per instruction, written to
//     the wave's LDS slice and read back in the score MFMA's A layout; the k_R operands
//     come straight from global memory in that layout (each lane's 16 bytes are 8
//     consecutive elements of one gathered row); the scores run on the bf16 MFMA against
//     the bf16 queries: all products exact;
//   - the 32 V_j rows are then gathered into the same slice (rows outside the list or
//     the sequence as zeros) and read back transposed as the A operand of
//     O^T += V^T P^T;
//   - P is split into two bf16 terms (hi + lo, about 16 significant bits) so that the
//     value contraction stays on the bf16 MFMA without rounding P to 8 bits.
// fp32 kernel: one workgroup per (chunk, sequence, query row), scores in LDS.
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

constexpr int DH = 128;   // per-group key/value width
constexpr int DR = 64;    // rotary key width
constexpr int TT = 32;    // listed rows per tile
constexpr int VSTRIDE = DH + 16;   // LDS row stride of the V tile: 72 dwords = 8 x odd
constexpr int NWS = 4;             // independent waves per block
constexpr float kLazy = 10.f;      // see decode_absorb.hip: reference raised only by > 2^10

struct SoftmaxState {
    float m;   // reference (log2 domain), identical in the 4 lanes of a row
    float l;   // lane-partial running sum of 2^(s - m)
};

// sc: log2-domain scores of the lane's 8 slot tokens (masked: -inf).  Writes p (fp32,
// relative to the updated reference); need: the row had accumulated under its old
// reference and raised it, so its accumulators must be multiplied by alpha first.
__device__ __forceinline__ void softmax_tile(SoftmaxState& st, const float (&sc)[8], float (&p)[8], bool& need,
                                             float& alpha) {
    float mt = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mt = wave_max16x4(mt);
    const bool raise = mt > st.m + kLazy;
    need = raise && st.m != kNegInf;
    alpha = raise ? fast_exp2(st.m - mt) : 1.f;
    st.l *= alpha;
    st.m = raise ? mt : st.m;
    const float muse = (st.m == kNegInf) ? 0.f : st.m;
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(sc[e] - muse);
    st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

__global__ __launch_bounds__(NWS * 64) void gqa_sparse_kernel(
    const u16* __restrict__ q_nope, const u16* __restrict__ q_rope, const u16* __restrict__ cache,
    int64_t bstride, const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ indices, int topk,
    int max_ctx, int h_q, int g, int s_q, int chunk, int n_split, int batch, int RT, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
    __shared__ __attribute__((aligned(16))) u16 vt[NWS][TT * VSTRIDE];
    __shared__ int idx_lds[NWS][TT];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int n_items = batch * s_q * g * RT * n_split;
    const int item = blockIdx.x * NWS + wave;
    if (item >= n_items) return;      // no block barrier below: idle waves may leave
    int rem = item;
    const int p = rem % n_split;
    rem /= n_split;
    const int rt = rem % RT;
    rem /= RT;
    const int j = rem % g;
    rem /= g;
    const int s = rem % s_q;
    const int b = rem / s_q;

    const int hpg = h_q / g;
    const int hh = rt * 16 + r16;
    const bool row_ok = hh < hpg;
    const int h = j * hpg + (row_ok ? hh : 0);
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int nvis = clampi(L - s_q + s + 1, 0, L);
    const int W = 2 * g * DH + DR;
    const int k0 = p * chunk, k1 = min(k0 + chunk, topk);
    const int32_t* ilist = indices + ((size_t)(b * s_q + s) * g + j) * topk;
    const u16* seq = cache + (size_t)b * bstride;
    const size_t qrow = ((size_t)b * s_q + s) * h_q + h;

    // queries as the B operand of S^T = K Q^T: k-steps 0..3 over q^N, 4..5 over q^R
    bf16x8 qv[6];
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) {
        const u16* src = kk < 4 ? q_nope + qrow * DH + kk * 32 + q4 * 8 : q_rope + qrow * DR + (kk - 4) * 32 + q4 * 8;
        qv[kk] = row_ok ? ld_bf16x8(src) : zero_bf16x8();
    }
    floatx4 oacc[DH / 16];
#pragma unroll
    for (int n = 0; n < DH / 16; ++n) oacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    SoftmaxState st{kNegInf, 0.f};
    u16* vl = vt[wave];
    int* il = idx_lds[wave];

    // The tile's 32 indices go through the wave's LDS slice; the next tile's are loaded one
    // tile ahead.  Every row load below is unconditional (rows outside the sequence read
    // row 0 and are zeroed or masked afterwards), so the compiler issues all of a tile's
    // loads before it waits for any.
    int next_idx = (lane < TT && k0 + lane < k1) ? ilist[k0 + lane] : -1;
    for (int kb = k0; kb < k1; kb += TT) {
        if (lane < TT) il[lane] = next_idx;
        next_idx = (lane < TT && kb + TT + lane < k1) ? ilist[kb + TT + lane] : -1;
        // LDS operations of one wave complete in order: the reads below see these writes
        const int t0 = il[r16], t1 = il[16 + r16];
        const u16* row0 = seq + (size_t)((t0 >= 0 && t0 < L) ? t0 : 0) * W;
        const u16* row1 = seq + (size_t)((t1 >= 0 && t1 < L) ? t1 : 0) * W;
        constexpr int NV = TT * (DH / 8) / 64;
        // K_j rows of the tile: lane piece c = k * 64 + lane is row c / 16, 8 columns
        // (c % 16) * 8, so that an instruction gathers 4 rows x 256 bytes.  Loaded in the
        // score MFMA's own layout (16 rows x 64 bytes per instruction), random rows gather
        // at about 0.8 of that rate on MI355X; the rows reach that layout through the wave's
        // LDS slice instead.  Nontemporal, as V_j below.  k_R (two k-steps) keeps the MFMA
        // layout and the default policy: the other groups' lists read it too, mostly from L2.
        u32x4 kv[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int c = k * 64 + lane;
            const int t = il[c >> 4];
            kv[k] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(seq + (size_t)((t >= 0 && t < L) ? t : 0) * W + j * DH + (c & 15) * 8));
        }
        bf16x8 ka[6], kc[6];
#pragma unroll
        for (int kk = 4; kk < 6; ++kk) {
            const int col = 2 * g * DH + (kk - 4) * 32 + q4 * 8;
            ka[kk] = ld_bf16x8(row0 + col);
            kc[kk] = ld_bf16x8(row1 + col);
        }
        // V_j rows of the tile: chunk c = 16 per row.  Nontemporal: a V_j (or K_j) row
        // belongs to one group and is not read again this step (on MI355X 234 -> 217 us at
        // 2048 rows per (b, j) for V_j; with K_j too, and K_j through LDS, 212 -> 194 us).
        u32x4 vv[NV];
        bool vok[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int c = k * 64 + lane;
            const int t = il[c >> 4];
            vok[k] = t >= 0 && t < L;
            vv[k] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(seq + (size_t)(vok[k] ? t : 0) * W + (g + j) * DH + (c & 15) * 8));
        }
        // K_j into the slice and back in the MFMA layout (rows 0..15, then 16..31)
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int c = k * 64 + lane;
            *reinterpret_cast<u32x4*>(vl + (c >> 4) * VSTRIDE + (c & 15) * 8) = kv[k];
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            ka[kk] = ld_bf16x8(vl + r16 * VSTRIDE + kk * 32 + q4 * 8);
            kc[kk] = ld_bf16x8(vl + (16 + r16) * VSTRIDE + kk * 32 + q4 * 8);
        }
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) {
            acc0 = mfma16(ka[kk], qv[kk], acc0);
            acc1 = mfma16(kc[kk], qv[kk], acc1);
        }
        // V_j into the same slice (after the K_j reads above: one wave's LDS operations
        // complete in order), rows outside the list or the sequence as zeros
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int c = k * 64 + lane;
            *reinterpret_cast<u32x4*>(vl + (c >> 4) * VSTRIDE + (c & 15) * 8) = vok[k] ? vv[k] : u32x4{0u, 0u, 0u, 0u};
        }
        // scores of the lane's slot tokens 16(e/4) + 4q4 + e%4 (the D layout of S^T)
        float sc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = il[16 * (e >> 2) + 4 * q4 + (e & 3)];
            const float v = (e < 4 ? acc0 : acc1)[e & 3];
            sc[e] = (row_ok && t >= 0 && t < nvis) ? v * scale_log2 : kNegInf;
        }
        float pr[8];
        bool need;
        float alpha;
        softmax_tile(st, sc, pr, need, alpha);
        if (__builtin_expect(__any(need), 0)) {
#pragma unroll
            for (int n = 0; n < DH / 16; ++n) oacc[n] *= alpha;
        }
        u32x4 ph, pl;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const u16 a = f2bf(pr[2 * k]), c = f2bf(pr[2 * k + 1]);
            ph[k] = pack2(a, c);
            pl[k] = pack2f(pr[2 * k] - bf2f(a), pr[2 * k + 1] - bf2f(c));
        }
        const bf16x8 pbh = as_bf16x8(ph), pbl = as_bf16x8(pl);
#pragma unroll
        for (int n = 0; n < DH / 16; ++n) {
            // A operand: column 16n + r16 of the V tile at the lane's eight slot tokens
            const u16* p0 = vl + (4 * q4 + (r16 >> 2)) * VSTRIDE + 16 * n + 4 * (r16 & 3);
            const u32x2 lo = lds_read_tr16(p0);
            const u32x2 hi = lds_read_tr16(p0 + 16 * VSTRIDE);
            const bf16x8 a = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            oacc[n] = mfma16(a, pbh, oacc[n]);
            oacc[n] = mfma16(a, pbl, oacc[n]);
        }
    }
    if (!row_ok) return;
    const float l = wave_sum16x4(st.l);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t prow = ((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h;
    float* po = part_o + prow * DH;
#pragma unroll
    for (int n = 0; n < DH / 16; ++n) *reinterpret_cast<floatx4*>(po + 16 * n + 4 * q4) = oacc[n] * inv;
    if (q4 == 0) part_lse[prow] = l > 0.f ? (st.m + __log2f(l)) * kLn2 : kNegInf;
}

// fp32: grid = (n_split, batch, s_q*h_q); query row rho = s*h_q + h
constexpr int NT32 = 256;

__global__ __launch_bounds__(NT32) void gqa_sparse_f32_kernel(
    const float* __restrict__ q_nope, const float* __restrict__ q_rope, const float* __restrict__ cache,
    int64_t bstride, const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ indices, int topk,
    int max_ctx, int h_q, int g, int s_q, int d_r, int d_h, int chunk, int batch, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
    __shared__ float qv[256 + 256];
    __shared__ float sc[kF32MaxChunk];
    __shared__ int rows[kF32MaxChunk];
    __shared__ float red[NT32 / 64];
    const int p = blockIdx.x, b = blockIdx.y, rho = blockIdx.z;
    const int s = rho / h_q, h = rho - s * h_q;
    const int j = h / (h_q / g);
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int nvis = clampi(L - s_q + s + 1, 0, L);
    const int W = 2 * g * d_h + d_r;
    const int k0 = p * chunk, k1 = min(k0 + chunk, topk);
    const int n = max(k1 - k0, 0);
    const int32_t* ilist = indices + ((size_t)(b * s_q + s) * g + j) * topk;
    const size_t qrow = ((size_t)b * s_q + s) * h_q + h;
    const int tid = threadIdx.x;
    for (int k = tid; k < d_h + d_r; k += NT32) qv[k] = k < d_h ? q_nope[qrow * d_h + k] : q_rope[qrow * d_r + (k - d_h)];
    __syncthreads();
    const float* seq = cache + (size_t)b * bstride;
    for (int k = tid; k < n; k += NT32) {
        const int t = ilist[k0 + k];
        const bool ok = t >= 0 && t < nvis;
        rows[k] = ok ? t : -1;
        float acc = 0.f;
        if (ok) {
            const float* row = seq + (size_t)t * W;
            for (int d = 0; d < d_h; ++d) acc += qv[d] * row[j * d_h + d];
            for (int e = 0; e < d_r; ++e) acc += qv[d_h + e] * row[2 * g * d_h + e];
        }
        sc[k] = ok ? acc * scale_log2 : kNegInf;
    }
    __syncthreads();
    float mx = kNegInf;
    for (int k = tid; k < n; k += NT32) mx = fmaxf(mx, sc[k]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    float m = red[0];
    for (int w = 1; w < NT32 / 64; ++w) m = fmaxf(m, red[w]);
    __syncthreads();
    const float muse = m == kNegInf ? 0.f : m;
    float sum = 0.f;
    for (int k = tid; k < n; k += NT32) {
        const float pv = exp2f(sc[k] - muse);
        sc[k] = pv;
        sum += pv;
    }
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if ((tid & 63) == 0) red[tid >> 6] = sum;
    __syncthreads();
    float l = 0.f;
    for (int w = 0; w < NT32 / 64; ++w) l += red[w];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t prow = ((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h;
    for (int d = tid; d < d_h; d += NT32) {
        float acc = 0.f;
        for (int k = 0; k < n; ++k)
            if (rows[k] >= 0) acc += sc[k] * seq[(size_t)rows[k] * W + (g + j) * d_h + d];
        part_o[prow * d_h + d] = acc * inv;
    }
    if (tid == 0) part_lse[prow] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_gqa_sparse(const DecodeArgs& a, const int32_t* indices, int topk, bool bf16, hipStream_t st) {
    hipError_t e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    if (bf16) {
        const int hpg = a.h_q / a.g;
        const int RT = (hpg + 15) / 16;
        const int items = a.batch * a.s_q * a.g * RT * a.n_split;
        hipLaunchKernelGGL(gqa_sparse_kernel, dim3((items + NWS - 1) / NWS), dim3(NWS * 64), 0, st,
                           (const u16*)a.q_nope, (const u16*)a.q_rope, (const u16*)a.cache, a.bstride, a.ctx_lens,
                           indices, topk, a.max_ctx, a.h_q, a.g, a.s_q, a.chunk, a.n_split, a.batch, RT,
                           a.scale * kLog2e, a.part_o, a.part_lse);
    } else {
        dim3 grid(a.n_split, a.batch, a.s_q * a.h_q);
        hipLaunchKernelGGL(gqa_sparse_f32_kernel, grid, dim3(NT32), 0, st, (const float*)a.q_nope,
                           (const float*)a.q_rope, (const float*)a.cache, a.bstride, a.ctx_lens, indices, topk,
                           a.max_ctx, a.h_q, a.g, a.s_q, a.d_r, a.d_h, a.chunk, a.batch, a.scale * kLog2e, a.part_o,
                           a.part_lse);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

}  // namespace gqla
