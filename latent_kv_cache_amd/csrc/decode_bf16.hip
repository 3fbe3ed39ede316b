// bf16 MFMA decode kernels for gfx950: GQA path and MQA-absorb path.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Architecture).  Both paths compute,
// per sequence b, query token s and head i of group j = i / (h_q/g), softmax
// attention over the visible cached tokens t <= L_b - s_q + s:
//   GQA:    score_t = scale [q^N | q^R].[K_j,t | k_R,t],  o = sum_t p_t V_j,t
//   absorb: score_t = scale [W_UK[j]^T q^N | q^R].[c_t | k_R,t],
//           o = W_UV[j] sum_t p_t c_t
// over one context chunk per workgroup (split-K).  Each workgroup writes the
// chunk's normalised output and its log-sum-exp; launch_combine merges them.
//
// Tiling.  A workgroup streams its chunk in tiles of 32 cache rows.  A tile is
// one contiguous span of HBM (rows of a sequence are packed), loaded with
// 16-byte vector loads into registers one tile ahead and stored into LDS with
// a 32-byte pad per row.  On gfx950 a row stride of 8 x (odd) dwords modulo the 64
// LDS banks lets the 16-byte operand reads of 16 rows, and the transposing reads of
// 4 rows x 32 bytes, proceed at close to the full LDS rate (a 16-byte pad, 36 dwords
// mod 64, measured at about 60 % of it).
// HBM holds bf16; the tile is converted to fp16 on its way into LDS (exact for
// bf16 values within fp16's range) and the contractions run on fp16 MFMA, so the
// absorbed query and the softmax weights P, which the kernel itself rounds, keep
// 10 mantissa bits instead of 7.
// Each wave owns 16 query rows (the M = 16 side of the 16x16x32 MFMA: the 16
// heads of a group on the GQA path at h_q/g = 16, or 16 of the heads sharing
// the latent on the absorb path) and keeps its queries and accumulators in
// registers:
//   S^T[token][row] = K_tile . Q^T   (A = cache rows from LDS, B = queries)
//   O^T[feat][row] += V_tile^T . P^T (A = cache columns from LDS, B = P)
// so the softmax state of a row lives in the four lanes l%16 + 16q.
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

constexpr int DH = 128;   // per-group key/value width
constexpr int DR = 64;    // rotary key width
constexpr int RK = 512;   // latent width
constexpr int TT = 32;    // tokens per tile

// Token held by k-slot e (0..7) of lane group q (0..3) in the P / V^T operands:
// the softmax keeps S for tokens 16*(e/4) + 4q + (e%4), the D-layout of the two
// 16-token halves of S^T.
__device__ __forceinline__ int slot_token(int q, int e) { return 16 * (e >> 2) + 4 * q + (e & 3); }

// Online softmax with a lazily raised reference.  Exponentials are taken against a
// per-row reference m (log2 domain) that is raised only when a tile's maximum exceeds
// it by more than kLazy; otherwise p = 2^(s - m) <= 2^kLazy, which fp16 P and fp32
// sums hold as precisely as values <= 1.  When no row of the wave raises its
// reference, the accumulators need no rescaling for that tile.  The final
// normalisation and log-sum-exp use the same reference, so the result is that of
// the exact softmax.
constexpr float kLazy = 10.f;

struct SoftmaxState {
    float m;   // reference (log2 domain), identical in the 4 lanes of a row; -inf before any row
    float l;   // lane-partial running sum of 2^(s - m)
};

// sc[e] are log2-scaled scores for slot_token(q4, e), masked slots -inf.  Returns P as
// the fp16 B operand; sets rescale (wave-uniform) and alpha when accumulators must be
// multiplied by alpha before this tile's P is added.
__device__ __forceinline__ f16x8 softmax_tile(SoftmaxState& st, float (&sc)[8], bool& rescale, float& alpha) {
    float mt = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sc[e]);
    mt = wave_max16x4(mt);
    const bool raise = mt > st.m + kLazy;        // false while the row has seen nothing
    rescale = __any(raise);
    alpha = 1.f;
    if (raise) {
        alpha = fast_exp2(st.m - mt);            // st.m = -inf gives 0
        st.l *= alpha;
        st.m = mt;
    }
    const float muse = (st.m == kNegInf) ? 0.f : st.m;
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(sc[e] - muse);
        ps += p[e];
    }
    st.l += ps;
    u32x4 pk;
    pk[0] = pack2h(p[0], p[1]);
    pk[1] = pack2h(p[2], p[3]);
    pk[2] = pack2h(p[4], p[5]);
    pk[3] = pack2h(p[6], p[7]);
    return as_f16x8(pk);
}

// A operand of O^T += V^T P^T: lane (q4, r16) needs column col0 + r16 of the tile at
// the eight slot tokens 4q4 + e and 16 + 4q4 + e (e = 0..3).  Lane m of the 16-lane
// group addresses row 4q4 + m/4 (then 16 rows further), columns col0 + 4(m%4)..+3;
// the transposing read hands lane j column col0 + j of those rows.
__device__ __forceinline__ f16x8 gather_col(const u16* lds, int stride, int q4, int r16, int col0) {
    const u16* p0 = lds + (4 * q4 + (r16 >> 2)) * stride + col0 + 4 * (r16 & 3);
    const u32x2 lo = lds_read_tr16(p0);
    const u32x2 hi = lds_read_tr16(p0 + 16 * stride);
    return as_f16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Copy rows [row0, row0 + nrows) of a packed row-major span (width W elements) into
// registers: chunk c = tid + k*NT of the tile, 16 bytes each.  Rows past nrows load zeros.
template <int W, int NT, int NLOAD>
__device__ __forceinline__ void load_tile(u32x4 (&reg)[NLOAD], const u16* __restrict__ base, int nrows, int tid) {
    constexpr int CPR = W / 8;   // 16-byte chunks per row
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
        const int c = tid + k * NT;
        const int r = c / CPR;
        if (c < TT * CPR && r < nrows) {
            reg[k] = *reinterpret_cast<const u32x4*>(base + (size_t)c * 8);
        } else {
            reg[k] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// Store the staged tile into LDS as fp16 (bf16 -> fp16 conversion per element).
template <int W, int STRIDE, int NT, int NLOAD>
__device__ __forceinline__ void store_tile(u16* lds, const u32x4 (&reg)[NLOAD], int tid) {
    constexpr int CPR = W / 8;
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
        const int c = tid + k * NT;
        if (c < TT * CPR) {
            const int r = c / CPR;
            const int col = c - r * CPR;
            *reinterpret_cast<u32x4*>(lds + r * STRIDE + col * 8) = bf8_to_h8(reg[k]);
        }
    }
}

// ---------------------------------------------------------------------------
// GQA decode.  grid = (n_split, batch, pair blocks); block = NW waves.  The
// (group, 16-row tile) pairs of a sequence are numbered pair = j*RT + rt with
// RT = ceil(rows_per_group / 16); block z handles pairs [z*NW, z*NW + NW).
// Rows of group j are numbered rho = s*hpg + hh (query token s, head j*hpg + hh).
// ---------------------------------------------------------------------------
template <int G, int NW>
__global__ __launch_bounds__(NW * 64) void gqa_decode_kernel(
    const u16* __restrict__ q_nope, const u16* __restrict__ q_rope,
    const u16* __restrict__ cache, int64_t bstride, const int32_t* __restrict__ ctx_lens,
    int max_ctx, int h_q, int s_q, int chunk, int batch, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
    constexpr int W = 2 * G * DH + DR;
    constexpr int STRIDE = W + 16;   // row stride = 8 x odd dwords mod 64 banks
    constexpr int NT = NW * 64;
    constexpr int NLOAD = (TT * (W / 8) + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) u16 lds[TT * STRIDE];

    const int p = blockIdx.x, b = blockIdx.y;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int t0 = p * chunk;
    if (t0 >= L) return;                      // uniform over the block
    const int t1 = min(t0 + chunk, L);
    const int ntiles = (t1 - t0 + TT - 1) / TT;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int hpg = h_q / G;
    const int rows_g = s_q * hpg;
    const int RT = (rows_g + 15) >> 4;
    const int pair = blockIdx.z * NW + wave;
    const bool active = pair < G * RT;
    const int j = active ? pair / RT : 0;
    const int rt = active ? pair - j * RT : 0;
    const int rho = rt * 16 + r16;
    const bool row_ok = active && rho < rows_g;
    const int s = row_ok ? rho / hpg : 0;
    const int h = j * hpg + (row_ok ? rho - s * hpg : 0);
    const int nvis = clampi(L - s_q + s + 1, 0, L);
    const int qrow = (b * s_q + s) * h_q + h;

    // queries as the B operand of S^T = K Q^T: k-steps 0..3 over q^N, 4..5 over q^R
    f16x8 qv[6];
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) {
        if (row_ok) {
            const u16* src = kk < 4 ? q_nope + (size_t)qrow * DH + kk * 32 + q4 * 8
                                    : q_rope + (size_t)qrow * DR + (kk - 4) * 32 + q4 * 8;
            qv[kk] = as_f16x8(bf8_to_h8(*reinterpret_cast<const u32x4*>(src)));
        } else {
            qv[kk] = zero_f16x8();
        }
    }

    floatx4 oacc[DH / 16];
#pragma unroll
    for (int n = 0; n < DH / 16; ++n) oacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    SoftmaxState st{kNegInf, 0.f};

    const u16* seq = cache + (size_t)b * bstride;
    u32x4 reg[NLOAD];
    load_tile<W, NT, NLOAD>(reg, seq + (size_t)t0 * W, min(TT, t1 - t0), tid);

    for (int it = 0; it < ntiles; ++it) {
        const int tb = t0 + it * TT;
        if (it > 0) __syncthreads();
        store_tile<W, STRIDE, NT, NLOAD>(lds, reg, tid);
        __syncthreads();
        if (it + 1 < ntiles) {
            const int tn = tb + TT;
            load_tile<W, NT, NLOAD>(reg, seq + (size_t)tn * W, min(TT, t1 - tn), tid);
        }
        if (!active) continue;

        float sc[8];
        {
            // two independent accumulator chains per 16-token half
            floatx4 acc[2][2] = {};
#pragma unroll
            for (int kk = 0; kk < 6; ++kk) {
                const int col = kk < 4 ? j * DH + kk * 32 + q4 * 8 : 2 * G * DH + (kk - 4) * 32 + q4 * 8;
#pragma unroll
                for (int th = 0; th < 2; ++th)
                    acc[th][kk & 1] = mfma16h(ld_f16x8(lds + (th * 16 + r16) * STRIDE + col), qv[kk], acc[th][kk & 1]);
            }
#pragma unroll
            for (int th = 0; th < 2; ++th) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = tb + th * 16 + q4 * 4 + i;
                    const float v = acc[th][0][i] + acc[th][1][i];
                    sc[th * 4 + i] = (row_ok && t < t1 && t < nvis) ? v * scale_log2 : kNegInf;
                }
            }
        }
        bool rescale;
        float alpha;
        const f16x8 pb = softmax_tile(st, sc, rescale, alpha);
        if (__builtin_expect(rescale, 0)) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int n = 0; n < DH / 16; ++n) oacc[n] *= alpha;
        }
        const int vcol = (G + j) * DH;
#pragma unroll
        for (int n = 0; n < DH / 16; ++n)
            oacc[n] = mfma16h(gather_col(lds, STRIDE, q4, r16, vcol + 16 * n), pb, oacc[n]);
    }
    if (!row_ok) return;

    const float l = wave_sum16x4(st.l);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t prow = ((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h;
    float* po = part_o + prow * DH;
#pragma unroll
    for (int n = 0; n < DH / 16; ++n) {
        *reinterpret_cast<floatx4*>(po + 16 * n + 4 * q4) = oacc[n] * inv;
    }
    if (q4 == 0) part_lse[prow] = l > 0.f ? (st.m + __log2f(l)) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------------------
// Absorb prologue: qhat[b][rho][0:512] = W_UK[j]^T q^N, qhat[b][rho][512:576] = q^R,
// rho = s*h_q + h, stored as fp16 (the operand type of the decode kernel's MFMA).
// grid = (row blocks of 64, g); block = 4 waves.  The rows of group j are numbered
// iota = (b*s_q + s)*hpg + hh.  W_UK[j] ([d][r], 128 KB) is staged row-major in LDS;
// the contraction runs over d, so the A operand (W_UK^T) is formed with transposing
// LDS reads: 4 rows d x 16 columns r per 16-lane group.
// ---------------------------------------------------------------------------
constexpr int PRO_STRIDE = RK + 16;

__global__ __launch_bounds__(256) void absorb_prologue_kernel(
    const u16* __restrict__ q_nope, const u16* __restrict__ q_rope, const u16* __restrict__ w_uk,
    u16* __restrict__ qhat, int batch, int h_q, int g, int s_q) {
    __shared__ __attribute__((aligned(16))) u16 wt[DH * PRO_STRIDE];
    const int j = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;

    const u16* wj = w_uk + (size_t)j * DH * RK;
    for (int c = tid; c < DH * (RK / 8); c += 256) {
        const int d = c >> 6, r8 = c & 63;
        *reinterpret_cast<u32x4*>(wt + d * PRO_STRIDE + r8 * 8) =
            *reinterpret_cast<const u32x4*>(wj + (size_t)d * RK + r8 * 8);
    }
    __syncthreads();

    const int hpg = h_q / g;
    const int nrows = batch * s_q * hpg;
    const int iota = blockIdx.x * 64 + wave * 16 + r16;
    const bool ok = iota < nrows;
    const int bs = ok ? iota / hpg : 0;
    const int hh = ok ? iota - bs * hpg : 0;
    const int b = bs / s_q, s = bs - (bs / s_q) * s_q;
    const int h = j * hpg + hh;
    const size_t qrow = ((size_t)b * s_q + s) * h_q + h;
    const int RQ = s_q * h_q;
    u16* dst = qhat + ((size_t)b * RQ + (size_t)s * h_q + h) * (RK + DR);

    bf16x8 qb[DH / 32];
#pragma unroll
    for (int kd = 0; kd < DH / 32; ++kd) qb[kd] = ok ? ld_bf16x8(q_nope + qrow * DH + kd * 32 + q4 * 8) : zero_bf16x8();

    // A operand lane (q4, r16), k-step kd: W_UK[32kd + 8q4 + e][16mt + r16], e = 0..7
    const u16* abase = wt + (8 * q4 + (r16 >> 2)) * PRO_STRIDE + 4 * (r16 & 3);
#pragma unroll 4
    for (int mt = 0; mt < RK / 16; ++mt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kd = 0; kd < DH / 32; ++kd) {
            const u16* pa = abase + kd * 32 * PRO_STRIDE + mt * 16;
            const u32x2 lo = lds_read_tr16(pa);
            const u32x2 hi = lds_read_tr16(pa + 4 * PRO_STRIDE);
            acc = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), qb[kd], acc);
        }
        if (ok) {
            u32x2 o;
            o[0] = pack2h(acc[0], acc[1]);
            o[1] = pack2h(acc[2], acc[3]);
            *reinterpret_cast<u32x2*>(dst + mt * 16 + q4 * 4) = o;
        }
    }
    if (ok) {
        // q^R: 64 elements = 8 chunks of 16 bytes; lane group q4 copies chunks q4 and q4 + 4
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int off = (q4 + 4 * c) * 8;
            *reinterpret_cast<u32x4*>(dst + RK + off) =
                bf8_to_h8(*reinterpret_cast<const u32x4*>(q_rope + qrow * DR + off));
        }
    }
}

// ---------------------------------------------------------------------------
// Absorb latent attention with fused W_UV.  Block = NW waves of 16 query rows each
// (rho = z*16NW + 16w + (0..15) of the s_q*h_q rows, rho = s*h_q + h), all
// attending to the shared 576-wide rows; each wave keeps its absorbed queries (72
// registers) and u (128 registers) for the whole chunk.
//
// Tiles of 32 rows reach LDS by direct global->LDS loads (global_load_lds_dwordx4:
// lane l of a wave instruction lands at base + 16 l), three buffers deep, so two
// tiles are in flight while one is computed and no registers stage data.  Buffer
// slot s (16 bytes) is row s / SROW, column chunk s % SROW of a padded row-major
// tile; pad slots, slots of rows past the chunk and the spare tail slots receive a
// dummy in-bounds chunk.  Each wave issues exactly NDMA loads per tile, so waiting
// for vmcnt <= NDMA (vmcnt 0 on the last tile) means its part of the tile has landed.
// After a barrier the block converts the tile to fp16 in place (zeroing rows past
// the chunk), and after a second barrier it computes.
//
// After the chunk, u = P.C / l stays in registers and each group present in the
// wave's rows applies W_UV[j] with MFMA, so the partial written is o_p (d_h wide).
//
// One-dimensional grid, XCD-aware: when s_q*h_q needs nz > 1 blocks per (chunk,
// sequence), the nz blocks get ids 8 apart (same XCD, dispatched back to back), so
// the second read of every row is an L2 hit.
// ---------------------------------------------------------------------------
// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at LDS byte address lds_base + 16 l; lds_base must be wave-uniform.  It is
// issued from inline assembly so that the compiler, which cannot tell which LDS bytes
// such a load writes, does not wait for all of them before every later LDS access;
// callers wait with wait_vmcnt<> before reading the destination.  All compiler-visible
// global loads of a kernel that uses it must be issued before it or waited for by an
// explicit wait_vmcnt<0>, since the compiler does not count these loads.
// The global address is a wave-uniform 64-bit base (SGPRs) plus a 32-bit per-lane byte
// offset, so a lane spends one VGPR on it.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(gbase)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt immediate on gfx9: vmcnt = bits [3:0] and [15:14]; expcnt and
    // lgkmcnt fields left at their maxima (no wait on them)
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void absorb_decode_kernel(
    const u16* __restrict__ qhat, const u16* __restrict__ w_uv,
    const u16* __restrict__ cache, int64_t bstride, const int32_t* __restrict__ ctx_lens,
    int max_ctx, int h_q, int g, int s_q, int chunk, int n_split, int nz, int batch, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
    constexpr int W = RK + DR;
    constexpr int STRIDE = W + 16;    // row stride = 8 x odd dwords mod 64 banks
    constexpr int SROW = STRIDE / 8;  // 16-byte slots per LDS row (72 data + 2 pad)
    constexpr int CPR = W / 8;        // data slots per row
    constexpr int KS = W / 32;        // 18 k-steps of the score contraction
    constexpr int NU = RK / 16;       // 32 latent column tiles of U^T
    constexpr int NT = NW * 64;
    constexpr int TSLOTS = TT * SROW;                  // slots of a tile
    constexpr int NDMA = (TSLOTS + NT - 1) / NT;       // DMA instructions per wave per tile
    constexpr int BSLOTS = NDMA * NT;                  // slots of a buffer (spare tail included)
    constexpr int NBUF = 3;
    constexpr int KL = RK / 32;                        // 16 latent k-steps: q~ in registers
    constexpr int QRS = DR + 16;                       // LDS row stride of the rotary queries
    // three separately declared buffers: with the tile loop unrolled by three every
    // access names a fixed buffer, so the compiler can tell that reading one buffer
    // does not depend on the direct loads still landing in the others
    __shared__ __attribute__((aligned(16))) u16 buf0[BSLOTS * 8];
    __shared__ __attribute__((aligned(16))) u16 buf1[BSLOTS * 8];
    __shared__ __attribute__((aligned(16))) u16 buf2[BSLOTS * 8];
    __shared__ __attribute__((aligned(16))) u16 qr_lds[NW * 16 * QRS];

    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int z = slot % nz;
    const int pair = (slot / nz) * 8 + xcd;
    if (pair >= n_split * batch) return;           // padding of the last group of 8
    const int b = pair / n_split, p = pair - b * n_split;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int t0 = p * chunk;
    if (t0 >= L) return;
    const int t1 = min(t0 + chunk, L);
    const int ntiles = (t1 - t0 + TT - 1) / TT;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int RQ = s_q * h_q;
    const int hpg = h_q / g;
    const int rho0 = z * (NW * 16) + wave * 16;
    const bool active = rho0 < RQ;
    const int rho = rho0 + r16;
    const bool row_ok = rho < RQ;
    const int s = row_ok ? rho / h_q : 0;
    const int h = row_ok ? rho - s * h_q : 0;
    const int nvis = clampi(L - s_q + s + 1, 0, L);

    const u16* seq = cache + (size_t)b * bstride + (size_t)t0 * W;
    // byte offset within a tile of the chunk each of this lane's DMA slots carries
    // (-1: pad or spare slot, which receives the tile's first chunk as a dummy)
    int dma_off[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int sl = (i * NW + wave) * 64 + lane;
        const int r = sl / SROW, c = sl - r * SROW;
        dma_off[i] = (sl < TSLOTS && c < CPR) ? (r * W + c * 8) * 2 : -1;
    }
    // issue the direct loads of tile `it` into the buffer at LDS byte address tbuf
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    auto dma_tile = [&](int it, uint32_t tbuf) {
        const u16* tsrc = seq + (size_t)it * TT * W;
        const int lim = min(TT, t1 - t0 - it * TT) * W * 2;   // rows past the chunk: dummy
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const uint32_t off = (dma_off[i] >= 0 && dma_off[i] < lim) ? (uint32_t)dma_off[i] : 0u;
            dma16(tsrc, off, tbuf + (uint32_t)((i * NW + wave_s) * 1024));
        }
    };

    // absorbed latent queries in registers; the 64 rotary columns of the block's rows
    // in LDS (read twice per tile), made visible by the first tile barrier
    f16x8 qv[KL];
    const u16* qsrc = qhat + ((size_t)b * RQ + rho) * W + q4 * 8;
#pragma unroll
    for (int kk = 0; kk < KL; ++kk) qv[kk] = row_ok ? ld_f16x8(qsrc + kk * 32) : zero_f16x8();
    for (int c = tid; c < NW * 16 * (DR / 8); c += NT) {
        const int r = c / (DR / 8), col = c - r * (DR / 8);
        const int qrow = z * (NW * 16) + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (qrow < RQ) v = *reinterpret_cast<const u32x4*>(qhat + ((size_t)b * RQ + qrow) * W + RK + col * 8);
        *reinterpret_cast<u32x4*>(qr_lds + r * QRS + col * 8) = v;
    }
    const u16* qr_row = qr_lds + (wave * 16 + r16) * QRS + q4 * 8;

    floatx4 uacc[NU];
#pragma unroll
    for (int n = 0; n < NU; ++n) uacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    SoftmaxState st{kNegInf, 0.f};

    // barrier without the compiler's memory fence (whose vmcnt(0) would drain the
    // direct loads still in flight): own LDS operations complete, then s_barrier
    auto block_sync = [&]() {
        asm volatile("" ::: "memory");
        // s_waitcnt lgkmcnt(0): vmcnt field at its maximum 63 (bits [3:0] and [15:14]),
        // expcnt at 7, lgkmcnt (bits [11:8]) at 0
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // convert this lane's own DMA slots of tile `it` (in the buffer at `lds`) to fp16 in
    // place once its loads have landed; slots of rows past the chunk, pads and spare
    // slots become zero.  No other lane touches these slots, so no barrier is needed
    // before it, and the barrier at the top of the next iteration publishes the result.
    auto convert_own = [&](int it, u16* lds) {
        const int lim = min(TT, t1 - t0 - it * TT) * W * 2;
        u32x4 v[NDMA];
#pragma unroll
        for (int i = 0; i < NDMA; ++i) v[i] = *reinterpret_cast<const u32x4*>(lds + ((i * NW + wave) * 64 + lane) * 8);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const bool keep = dma_off[i] >= 0 && dma_off[i] < lim;
            *reinterpret_cast<u32x4*>(lds + ((i * NW + wave) * 64 + lane) * 8) =
                keep ? bf8_to_h8(v[i]) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    // one tile: (barrier) start the loads of tile it+2, compute tile it, then wait for
    // this wave's loads of tile it+1 and convert them.  One barrier per tile: it marks
    // tile it converted by every wave and tile it-1 (whose buffer the new loads reuse)
    // consumed by every wave.
    auto step = [&](int it, u16* lds, uint32_t dma_buf, u16* next_lds) {
        const int tb = t0 + it * TT;
        block_sync();
        if (it + 2 < ntiles) dma_tile(it + 2, dma_buf);
        if (active) {
            float sc[8];
            {
                floatx4 acc[2] = {};
                const u16* arow = lds + r16 * STRIDE + q4 * 8;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const f16x8 bq = kk < KL ? qv[kk] : ld_f16x8(qr_row + (kk - KL) * 32);
                    acc[0] = mfma16h(ld_f16x8(arow + kk * 32), bq, acc[0]);
                    acc[1] = mfma16h(ld_f16x8(arow + 16 * STRIDE + kk * 32), bq, acc[1]);
                    // bound how far the scheduler hoists operand reads (register pressure)
                    if (kk % 6 == 5) __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int th = 0; th < 2; ++th) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = tb + th * 16 + q4 * 4 + i;
                        sc[th * 4 + i] = (row_ok && t < t1 && t < nvis) ? acc[th][i] * scale_log2 : kNegInf;
                    }
                }
            }
            bool rescale;
            float alpha;
            const f16x8 pb = softmax_tile(st, sc, rescale, alpha);
            if (__builtin_expect(rescale, 0)) {
                // rare (the reference rose by more than kLazy); kept as a real branch so the
                // accumulators are not touched by VALU on the common path
                asm volatile("" ::: "memory");
#pragma unroll
                for (int n = 0; n < NU; ++n) uacc[n] *= alpha;
            }
#pragma unroll
            for (int n = 0; n < NU; ++n) {
                uacc[n] = mfma16h(gather_col(lds, STRIDE, q4, r16, 16 * n), pb, uacc[n]);
                if (n % 8 == 7) __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (it + 1 < ntiles) {
            if (it + 2 < ntiles) wait_vmcnt<NDMA>();    // tile it+2's loads may stay in flight
            else wait_vmcnt<0>();
            convert_own(it + 1, next_lds);
        }
    };

    const uint32_t a0 = lds_addr(buf0), a1 = lds_addr(buf1), a2 = lds_addr(buf2);
    dma_tile(0, a0);
    if (ntiles > 1) dma_tile(1, a1);
    if (ntiles > 1) wait_vmcnt<NDMA>();
    else wait_vmcnt<0>();
    convert_own(0, buf0);
    for (int it = 0; it < ntiles; it += NBUF) {
        step(it, buf0, a2, buf1);
        if (it + 1 < ntiles) step(it + 1, buf1, a0, buf2);
        if (it + 2 < ntiles) step(it + 2, buf2, a1, buf0);
    }
    if (!active) return;

    const float l = wave_sum16x4(st.l);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // U^T as the B operand of o^T = W_UV[j] U^T: k-step ks covers latent columns
    // 32ks + slot_token(q4, e), which are uacc[2ks + e/4][e%4] of this lane.  u is
    // split into two bf16 terms (u = hi + lo to about 16 bits) so that W_UV, which is
    // bf16, multiplies it with no rounding of u beyond fp32's.
    bf16x8 ub[RK / 32], ul[RK / 32];
#pragma unroll
    for (int ks = 0; ks < RK / 32; ++ks) {
        u32x4 vh, vl;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const floatx4& src = uacc[2 * ks + (h >> 1)];
            const float a = src[2 * (h & 1)] * inv, c = src[2 * (h & 1) + 1] * inv;
            const u16 ah = f2bf(a), ch = f2bf(c);
            vh[h] = pack2(ah, ch);
            vl[h] = pack2f(a - bf2f(ah), c - bf2f(ch));
        }
        ub[ks] = as_bf16x8(vh);
        ul[ks] = as_bf16x8(vl);
    }
    const int jrow = h / hpg;
    const size_t prow = ((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h;
    // groups of the wave's rows: rows never straddle a query token when h_q % 16 == 0
    const int last = min(rho0 + 15, RQ - 1);
    const int jlo = (rho0 % h_q) / hpg, jhi = (last % h_q) / hpg;
    for (int jj = jlo; jj <= jhi; ++jj) {
        const u16* wj = w_uv + (size_t)jj * DH * RK;
#pragma unroll 2
        for (int mt = 0; mt < DH / 16; ++mt) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            const u16* wrow = wj + (size_t)(mt * 16 + r16) * RK + q4 * 4;
#pragma unroll
            for (int ks = 0; ks < RK / 32; ++ks) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(wrow + ks * 32);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(wrow + ks * 32 + 16);
                const bf16x8 wa = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
                acc = mfma16(wa, ub[ks], acc);
                acc = mfma16(wa, ul[ks], acc);
            }
            if (row_ok && jrow == jj) *reinterpret_cast<floatx4*>(part_o + prow * DH + mt * 16 + q4 * 4) = acc;
        }
    }
    if (row_ok && q4 == 0) part_lse[prow] = l > 0.f ? (st.m + __log2f(l)) * kLn2 : kNegInf;
}

template <int G, int NW>
hipError_t launch_gqa_t(const DecodeArgs& a, hipStream_t st) {
    const int rows_g = a.s_q * (a.h_q / a.g);
    const int pairs = G * ((rows_g + 15) / 16);
    dim3 grid(a.n_split, a.batch, (pairs + NW - 1) / NW);
    hipError_t e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gqa_decode_kernel<G, NW>), grid, dim3(NW * 64), 0, st,
                       (const u16*)a.q_nope, (const u16*)a.q_rope, (const u16*)a.cache, a.bstride,
                       a.ctx_lens, a.max_ctx, a.h_q, a.s_q, a.chunk, a.batch, a.scale * kLog2e,
                       a.part_o, a.part_lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

// 8 waves per block: with 1024-thread blocks the 128-register cap spills the
// staging registers; extra (group, row tile) pairs go to further blocks in z.
template <int G>
hipError_t launch_gqa_g(const DecodeArgs& a, hipStream_t st) {
    return launch_gqa_t<G, 8>(a, st);
}

}  // namespace

int absorb_waves(int query_rows) { return query_rows <= 32 ? 2 : (query_rows <= 64 ? 4 : 8); }

bool gqa_bf16_supported(int g, int rows_per_group) {
    return (g == 1 || g == 2 || g == 4 || g == 8) && rows_per_group >= 1;
}

hipError_t launch_gqa_bf16(const DecodeArgs& a, hipStream_t st) {
    switch (a.g) {
        case 1: return launch_gqa_g<1>(a, st);
        case 2: return launch_gqa_g<2>(a, st);
        case 4: return launch_gqa_g<4>(a, st);
        case 8: return launch_gqa_g<8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_absorb_bf16(const DecodeArgs& a, hipStream_t st) {
    const int hpg = a.h_q / a.g;
    const int rows_per_group = a.batch * a.s_q * hpg;
    dim3 pgrid((rows_per_group + 63) / 64, a.g);
    hipLaunchKernelGGL(absorb_prologue_kernel, pgrid, dim3(256), 0, st,
                       (const u16*)a.q_nope, (const u16*)a.q_rope, (const u16*)a.w_uk, (u16*)a.qhat,
                       a.batch, a.h_q, a.g, a.s_q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int RQ = a.s_q * a.h_q;
    const int nw = absorb_waves(RQ);
    const int nz = (RQ + 16 * nw - 1) / (16 * nw);
    const int pairs = a.n_split * a.batch;
    dim3 grid(((pairs + 7) / 8) * 8 * nz);
    e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
#define GQLA_ABSORB_LAUNCH(NWV)                                                                          \
    hipLaunchKernelGGL(absorb_decode_kernel<NWV>, grid, dim3(NWV * 64), 0, st, (const u16*)a.qhat,             \
                       (const u16*)a.w_uv, (const u16*)a.cache, a.bstride, a.ctx_lens, a.max_ctx, a.h_q, a.g,   \
                       a.s_q, a.chunk, a.n_split, nz, a.batch, a.scale * kLog2e, a.part_o, a.part_lse)
    if (nw == 2) {
        GQLA_ABSORB_LAUNCH(2);
    } else if (nw == 4) {
        GQLA_ABSORB_LAUNCH(4);
    } else {
        GQLA_ABSORB_LAUNCH(8);
    }
#undef GQLA_ABSORB_LAUNCH
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

}  // namespace gqla
