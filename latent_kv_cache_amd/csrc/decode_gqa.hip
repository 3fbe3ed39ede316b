// bf16 MFMA GQA decode kernels for gfx950.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Architecture, GQA path).  Per sequence b,
// query token s and head i of group j = i / (h_q/g), softmax attention over the
// visible cached tokens t <= L_b - s_q + s of the once-expanded group rows:
//   score_t = scale [q^N | q^R].[K_j,t | k_R,t],  o = sum_t p_t V_j,t
// over one context chunk per workgroup (split-K).  Each workgroup writes the chunk's
// normalised output and its log-sum-exp; launch_combine merges them.
//
// Tiling.  A workgroup streams its chunk in tiles of cache rows.  A tile is one
// contiguous span of HBM (rows of a sequence are packed), held in LDS with a 32-byte
// pad per row.  On gfx950 a row stride of 8 x (odd) dwords modulo the 64 LDS banks lets
// the 16-byte operand reads of 16 rows, and the transposing reads of 4 rows x 32 bytes,
// proceed at close to the full LDS rate (a 16-byte pad, 36 dwords mod 64, measured at
// about 60 % of it).  Two ways to fill it:
//   - gqa_decode_kernel: 16-byte vector loads into registers one (or two) 32-row tiles
//     ahead, converted from bf16 to fp16 on the way into LDS (exact for bf16 values
//     within fp16's range); both contractions run on fp16 MFMA;
//   - gqa_dma_kernel (below): loads straight into one of two LDS buffers, used there in
//     bf16: scores on the bf16 MFMA, value operands converted to fp16 in registers.
// Either way the softmax weights P, which the kernel itself rounds, are fp16 and keep
// 10 mantissa bits instead of bf16's 7.
// Each wave owns 16 query rows (the N = 16 side of the 16x16x32 MFMA: the 16 heads
// of a group at h_q/g = 16) and keeps its queries and accumulators in registers:
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
static_assert(kChunkAlign == kBf16TokenTile && kChunkAlign % TT == 0, "chunks are whole tiles");

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
// The loads are nontemporal: every expanded row is read exactly once per decode step, and
// on MI355X the streaming hint lifts this kernel from about 6.1 to 6.9 TB/s (same data,
// same results).
template <int W, int NT, int NLOAD, int ROWS = TT>
__device__ __forceinline__ void load_tile(u32x4 (&reg)[NLOAD], const u16* __restrict__ base, int nrows, int tid) {
    constexpr int CPR = W / 8;   // 16-byte chunks per row
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
        const int c = tid + k * NT;
        const int r = c / CPR;
        if (c < ROWS * CPR && r < nrows) {
            reg[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (size_t)c * 8));
        } else {
            reg[k] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// Store the staged tile into LDS as fp16 (bf16 -> fp16 conversion per element).
template <int W, int STRIDE, int NT, int NLOAD, int ROWS = TT>
__device__ __forceinline__ void store_tile(u16* lds, const u32x4 (&reg)[NLOAD], int tid) {
    constexpr int CPR = W / 8;
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
        const int c = tid + k * NT;
        if (c < ROWS * CPR) {
            const int r = c / CPR;
            const int col = c - r * CPR;
            *reinterpret_cast<u32x4*>(lds + r * STRIDE + col * 8) = bf8_to_h8(reg[k]);
        }
    }
}

// ---------------------------------------------------------------------------
// GQA decode.  One-dimensional XCD-aware grid; block = NW waves.  Block id i runs on
// XCD i % 8; its slot i / 8 gives the pair block z = slot % nz and the work item
// u = (slot / nz) * 8 + i % 8, which chunk_of_item maps to a (sequence, chunk).  So the
// nz blocks that read the same tiles are 8 ids apart (one XCD, dispatched together:
// the second read is an L2 hit), and consecutive items run on consecutive XCDs.
// The (group, 16-row tile) pairs of a sequence are numbered pair = j*RT + rt with
// RT = ceil(rows_per_group / 16).  A wave owns RPW consecutive row tiles of one group
// (RPW divides RT): its K_j and V_j operand reads from LDS then feed RPW MFMAs each,
// and with RPW = 2 the 16 pairs of s_q = 2 at 16 heads per group (or of 32 heads per
// group at s_q = 2, g = 4) fit one block, which reads every tile from HBM once.
// Block z handles waves units [z*NW, z*NW + NW) of the G * RT / RPW.
// Rows of group j are numbered rho = s*hpg + hh (query token s, head j*hpg + hh).
// ---------------------------------------------------------------------------
template <int G, int NW, int RPW, int AHEAD>
__global__ __launch_bounds__(NW * 64) void gqa_decode_kernel(
    const u16* __restrict__ q_nope, const u16* __restrict__ q_rope,
    const u16* __restrict__ cache, int64_t bstride, const int32_t* __restrict__ ctx_lens,
    int max_ctx, int h_q, int s_q, int chunk, int n_split, int nz, int cap, int batch, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
    constexpr int W = 2 * G * DH + DR;
    constexpr int STRIDE = W + 16;   // row stride = 8 x odd dwords mod 64 banks
    constexpr int NT = NW * 64;
    constexpr int NLOAD = (TT * (W / 8) + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) u16 lds[TT * STRIDE];

    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int zb = slot % nz;
    const int unit = (slot / nz) * 8 + xcd;
    if (unit >= n_split * batch) return;      // padding of the last group of 8
    int b, p, t0, t1;
    if (!chunk_of_item<NT>(unit, ctx_lens, batch, max_ctx, chunk, cap, reinterpret_cast<int*>(lds), b, p, t0, t1)) return;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    __syncthreads();                          // the item is known to every thread before the tile reuses LDS
    const int ntiles = (t1 - t0 + TT - 1) / TT;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int hpg = h_q / G;
    const int rows_g = s_q * hpg;
    const int RT = (rows_g + 15) >> 4;
    const int wu = zb * NW + wave;             // wave unit: RPW row tiles of one group
    const bool active = wu * RPW < G * RT;
    const int j = active ? (wu * RPW) / RT : 0;
    const int rt0 = active ? wu * RPW - j * RT : 0;
    bool row_ok[RPW];
    int nvis[RPW], qrow[RPW];
#pragma unroll
    for (int rg = 0; rg < RPW; ++rg) {
        const int rho = (rt0 + rg) * 16 + r16;
        row_ok[rg] = active && rho < rows_g;
        const int s = row_ok[rg] ? rho / hpg : 0;
        const int h = j * hpg + (row_ok[rg] ? rho - s * hpg : 0);
        nvis[rg] = clampi(L - s_q + s + 1, 0, L);
        qrow[rg] = (b * s_q + s) * h_q + h;
    }

    // the first tile's loads go out before the queries', so the two round trips to memory
    // overlap at the start of every item
    const u16* seq = cache + (size_t)b * bstride;
    u32x4 reg[AHEAD][NLOAD];
#pragma unroll
    for (int a = 0; a < AHEAD; ++a)
        if (a == 0 || a < ntiles) load_tile<W, NT, NLOAD>(reg[a], seq + (size_t)(t0 + a * TT) * W, min(TT, t1 - t0 - a * TT), tid);
    // queries as the B operand of S^T = K Q^T: k-steps 0..3 over q^N, 4..5 over q^R
    f16x8 qv[RPW][6];
#pragma unroll
    for (int rg = 0; rg < RPW; ++rg)
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) {
            if (row_ok[rg]) {
                const u16* src = kk < 4 ? q_nope + (size_t)qrow[rg] * DH + kk * 32 + q4 * 8
                                        : q_rope + (size_t)qrow[rg] * DR + (kk - 4) * 32 + q4 * 8;
                qv[rg][kk] = as_f16x8(bf8_to_h8(*reinterpret_cast<const u32x4*>(src)));
            } else {
                qv[rg][kk] = zero_f16x8();
            }
        }

    floatx4 oacc[RPW][DH / 16];
#pragma unroll
    for (int rg = 0; rg < RPW; ++rg)
#pragma unroll
        for (int n = 0; n < DH / 16; ++n) oacc[rg][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    SoftmaxState st[RPW];
#pragma unroll
    for (int rg = 0; rg < RPW; ++rg) st[rg] = SoftmaxState{kNegInf, 0.f};

    // Tile it leaves staging buffer it % AHEAD for LDS, and the buffer takes tile it + AHEAD.
    auto tile_step = [&](int it, u32x4 (&rb)[NLOAD]) {
        const int tb = t0 + it * TT;
        if (it > 0) __syncthreads();
        store_tile<W, STRIDE, NT, NLOAD>(lds, rb, tid);
        __syncthreads();
        if (it + AHEAD < ntiles) {
            const int tn = tb + AHEAD * TT;
            load_tile<W, NT, NLOAD>(rb, seq + (size_t)tn * W, min(TT, t1 - tn), tid);
        }
        if (!active) return;

        f16x8 pb[RPW];
        {
            // two independent accumulator chains per 16-token half and row tile
            floatx4 acc[RPW][2][2] = {};
#pragma unroll
            for (int kk = 0; kk < 6; ++kk) {
                const int col = kk < 4 ? j * DH + kk * 32 + q4 * 8 : 2 * G * DH + (kk - 4) * 32 + q4 * 8;
#pragma unroll
                for (int th = 0; th < 2; ++th) {
                    const f16x8 a = ld_f16x8(lds + (th * 16 + r16) * STRIDE + col);
#pragma unroll
                    for (int rg = 0; rg < RPW; ++rg)
                        acc[rg][th][kk & 1] = mfma16h(a, qv[rg][kk], acc[rg][th][kk & 1]);
                }
            }
#pragma unroll
            for (int rg = 0; rg < RPW; ++rg) {
                float sc[8];
#pragma unroll
                for (int th = 0; th < 2; ++th) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = tb + th * 16 + q4 * 4 + i;
                        const float v = acc[rg][th][0][i] + acc[rg][th][1][i];
                        sc[th * 4 + i] = (row_ok[rg] && t < t1 && t < nvis[rg]) ? v * scale_log2 : kNegInf;
                    }
                }
                bool rescale;
                float alpha;
                pb[rg] = softmax_tile(st[rg], sc, rescale, alpha);
                if (__builtin_expect(rescale, 0)) {
                    asm volatile("" ::: "memory");
#pragma unroll
                    for (int n = 0; n < DH / 16; ++n) oacc[rg][n] *= alpha;
                }
            }
        }
        const int vcol = (G + j) * DH;
#pragma unroll
        for (int n = 0; n < DH / 16; ++n) {
            const f16x8 a = gather_col(lds, STRIDE, q4, r16, vcol + 16 * n);
#pragma unroll
            for (int rg = 0; rg < RPW; ++rg) oacc[rg][n] = mfma16h(a, pb[rg], oacc[rg][n]);
        }
    };
    // unrolled by AHEAD so that every staging buffer is addressed statically
    for (int it = 0; it < ntiles; it += AHEAD) {
#pragma unroll
        for (int a = 0; a < AHEAD; ++a)
            if (a == 0 || it + a < ntiles) tile_step(it + a, reg[a]);
    }

#pragma unroll
    for (int rg = 0; rg < RPW; ++rg) {
        // the four lanes of a row share row_ok, so the reduction runs over active lanes
        if (!row_ok[rg]) continue;
        const float l = wave_sum16x4(st[rg].l);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const size_t prow = (size_t)p * batch * s_q * h_q + qrow[rg];
        float* po = part_o + prow * DH;
#pragma unroll
        for (int n = 0; n < DH / 16; ++n) *reinterpret_cast<floatx4*>(po + 16 * n + 4 * q4) = oacc[rg][n] * inv;
        if (q4 == 0) part_lse[prow] = l > 0.f ? (st[rg].m + __log2f(l)) * kLn2 : kNegInf;
    }
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// softmax_tile for one 16-token half: sc[i] is token 4q + i.  Returns P as the B operand
// of the 16x16x16 fp16 MFMA (16 tokens x 16 rows).

__device__ __forceinline__ f16x4 softmax_tile4(SoftmaxState& st, float (&sc)[4], bool& rescale, float& alpha) {
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = wave_max16x4(mt);
    const bool raise = mt > st.m + kLazy;
    rescale = __any(raise);
    alpha = 1.f;
    if (raise) {
        alpha = fast_exp2(st.m - mt);
        st.l *= alpha;
        st.m = mt;
    }
    const float muse = (st.m == kNegInf) ? 0.f : st.m;
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = fast_exp2(sc[e] - muse);
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
    return __builtin_bit_cast(f16x4, u32x2{pack2h(p[0], p[1]), pack2h(p[2], p[3])});
}

// ---------------------------------------------------------------------------
// Tiles fed by direct loads: gqa_dma_kernel<G, NW, RPW, TR>, TR = 16 or 32 cache rows
// per tile.  Tiles go from global memory straight into one of two LDS buffers
// (global_load_lds_dwordx4) and are used there as loaded, in bf16: no staging registers,
// no conversion pass through LDS and one barrier per tile.  At step k, after the barrier
// that published tile k (buffer k % 2), every wave issues its share of tile k + 1's loads
// into buffer (k + 1) % 2, whose last reader was step k - 1, computes tile k, and waits
// for its own loads.  So a tile's loads are in flight for a whole step, where the
// register-staged kernel above issues them only after the previous tile's LDS store.
// The scores run on the bf16 MFMA against the queries as given; the value operands are
// converted to fp16 in registers after the transposing read, so that P keeps fp16's 11
// bits.  At TR = 16 the value product is the 16x16x16 fp16 MFMA, whose B operand (16
// tokens x 16 rows) is the lane's own four softmax weights in the D layout of the score
// tile; at TR = 32 it is the 16x16x32 one, as in gqa_decode_kernel.  Two buffers of 32
// rows fit LDS up to g = 4; at g = 8 the tiles have 16 rows (2 x 68.6 KB).
// A buffer holds TR rows at a stride of W + 16 elements (8 x odd dwords modulo the 64
// banks), rounded up to whole 64-lane instructions of 16-byte slots; the two pad slots of
// a row and any spare slots load the row's (or the tile's) first 16 bytes, a line loaded
// anyway, and are never read.  Rows past the chunk load the tile's first row (finite data,
// masked, P = 0).  Grid, work split and outputs as gqa_decode_kernel.
// ---------------------------------------------------------------------------
template <int G, int NW, int RPW, int TR>
__global__ __launch_bounds__(NW * 64) void gqa_dma_kernel(
    const u16* __restrict__ q_nope, const u16* __restrict__ q_rope,
    const u16* __restrict__ cache, int64_t bstride, const int32_t* __restrict__ ctx_lens,
    int max_ctx, int h_q, int s_q, int chunk, int n_split, int nz, int cap, int batch, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
    static_assert(TR == 16 || TR == 32, "16- or 32-row tiles");
    static_assert(kChunkAlign % TR == 0, "chunks are whole tiles");
    constexpr int W = 2 * G * DH + DR;
    constexpr int STRIDE = W + 16;
    constexpr int SROW = STRIDE / 8;                       // 16-byte slots per LDS row
    constexpr int CPR = W / 8;                             // data slots per row
    constexpr int NINST = (TR * SROW + 63) / 64;           // 64-lane load instructions per tile
    constexpr int BSLOTS = NINST * 64;                     // slots per buffer (with the spare ones)
    constexpr int MI = (NINST + NW - 1) / NW;              // load instructions per wave (at most)
    constexpr int NH = TR / 16;                            // 16-token halves per tile
    static_assert((STRIDE / 2) % 64 % 16 == 8, "row stride is 8 x odd dwords modulo 64 banks");
    __shared__ __attribute__((aligned(16))) u16 lds[2 * BSLOTS * 8];

    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int zb = slot % nz;
    const int unit = (slot / nz) * 8 + xcd;
    if (unit >= n_split * batch) return;
    int b, p, t0, t1;
    if (!chunk_of_item<NW * 64>(unit, ctx_lens, batch, max_ctx, chunk, cap, reinterpret_cast<int*>(lds), b, p, t0, t1))
        return;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    __syncthreads();                          // the item is known to every thread before the tiles reuse LDS
    const int ntiles = (t1 - t0 + TR - 1) / TR;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q4 = lane >> 4, r16 = lane & 15;
    const int hpg = h_q / G;
    const int rows_g = s_q * hpg;
    const int RT = (rows_g + 15) >> 4;
    const int wu = zb * NW + wave;
    const bool active = wu * RPW < G * RT;
    const int j = active ? (wu * RPW) / RT : 0;
    const int rt0 = active ? wu * RPW - j * RT : 0;
    bool row_ok[RPW];
    int nvis[RPW], qrow[RPW];
#pragma unroll
    for (int rg = 0; rg < RPW; ++rg) {
        const int rho = (rt0 + rg) * 16 + r16;
        row_ok[rg] = active && rho < rows_g;
        const int s = row_ok[rg] ? rho / hpg : 0;
        const int h = j * hpg + (row_ok[rg] ? rho - s * hpg : 0);
        nvis[rg] = clampi(L - s_q + s + 1, 0, L);
        qrow[rg] = (b * s_q + s) * h_q + h;
    }

    // Byte offset within a tile of the 16 bytes that slot (wave + NW m) * 64 + lane of a
    // buffer carries; instruction wave + NW m exists for m < MI - 1 and, for the first
    // NINST % NW waves (or all when it divides), for m = MI - 1.
    const u16* seq = cache + (size_t)b * bstride;
    uint32_t off[MI];
#pragma unroll
    for (int m = 0; m < MI; ++m) {
        const int sl = (wave + NW * m) * 64 + lane;
        const int r = sl / SROW, c = sl - (sl / SROW) * SROW;
        off[m] = (sl < TR * SROW) ? (uint32_t)((r * W + (c < CPR ? c : 0) * 8) * 2) : 0u;
    }
    const bool last_inst = (wave + NW * (MI - 1)) < NINST;
    const uint32_t lbase = lds_addr(lds);
    auto dma_tile = [&](int it) {
        const u16* tsrc = seq + (size_t)(t0 + it * TR) * W;
        const uint32_t tbuf = lbase + (uint32_t)((it & 1) * BSLOTS * 16);
        const int rows = t1 - t0 - it * TR;
        const uint32_t lim = rows >= TR ? 0xffffffffu : (uint32_t)(rows * W * 2);
#pragma unroll
        for (int m = 0; m < MI; ++m) {
            if (m < MI - 1 || last_inst) {
                const uint32_t o = off[m] < lim ? off[m] : off[m] % (uint32_t)(W * 2);
                dma16_nt(tsrc, o, tbuf + (uint32_t)((wave + NW * m) * 1024));
            }
        }
    };
    dma_tile(0);

    // queries as the B operand of S^T = K Q^T: k-steps 0..3 over q^N, 4..5 over q^R
    bf16x8 qv[RPW][6];
#pragma unroll
    for (int rg = 0; rg < RPW; ++rg)
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) {
            if (row_ok[rg]) {
                const u16* src = kk < 4 ? q_nope + (size_t)qrow[rg] * DH + kk * 32 + q4 * 8
                                        : q_rope + (size_t)qrow[rg] * DR + (kk - 4) * 32 + q4 * 8;
                qv[rg][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(src));
            } else {
                qv[rg][kk] = zero_bf16x8();
            }
        }

    floatx4 oacc[RPW][DH / 16];
#pragma unroll
    for (int rg = 0; rg < RPW; ++rg)
#pragma unroll
        for (int n = 0; n < DH / 16; ++n) oacc[rg][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    SoftmaxState st[RPW];
#pragma unroll
    for (int rg = 0; rg < RPW; ++rg) st[rg] = SoftmaxState{kNegInf, 0.f};

    for (int it = 0; it < ntiles; ++it) {
        // this wave's loads of tile it have landed (nothing else of it is in flight), and
        // after the barrier everyone's have, and tile it - 1's buffer is free
        wait_vmcnt<0>();
        block_sync();
        if (it + 1 < ntiles) dma_tile(it + 1);
        if (!active) continue;
        const int tb = t0 + it * TR;
        const u16* tile = lds + (it & 1) * BSLOTS * 8;

        f16x4 pb4[RPW];
        f16x8 pb8[RPW];
        {
            // two independent accumulator chains per 16-token half and row tile
            floatx4 acc[RPW][NH][2] = {};
#pragma unroll
            for (int kk = 0; kk < 6; ++kk) {
                const int col = kk < 4 ? j * DH + kk * 32 + q4 * 8 : 2 * G * DH + (kk - 4) * 32 + q4 * 8;
#pragma unroll
                for (int th = 0; th < NH; ++th) {
                    const bf16x8 a = ld_bf16x8(tile + (th * 16 + r16) * STRIDE + col);
#pragma unroll
                    for (int rg = 0; rg < RPW; ++rg)
                        acc[rg][th][kk & 1] = mfma16(a, qv[rg][kk], acc[rg][th][kk & 1]);
                }
            }
#pragma unroll
            for (int rg = 0; rg < RPW; ++rg) {
                float sc[4 * NH];
#pragma unroll
                for (int th = 0; th < NH; ++th)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = tb + th * 16 + q4 * 4 + i;
                        const float v = acc[rg][th][0][i] + acc[rg][th][1][i];
                        sc[th * 4 + i] = (row_ok[rg] && t < t1 && t < nvis[rg]) ? v * scale_log2 : kNegInf;
                    }
                bool rescale;
                float alpha;
                if constexpr (TR == 16) pb4[rg] = softmax_tile4(st[rg], sc, rescale, alpha);
                else pb8[rg] = softmax_tile(st[rg], sc, rescale, alpha);
                if (__builtin_expect(rescale, 0)) {
                    asm volatile("" ::: "memory");
#pragma unroll
                    for (int n = 0; n < DH / 16; ++n) oacc[rg][n] *= alpha;
                }
            }
        }
        // A operand: feature (G + j) d_h + 16n + r16 at the lane's slot tokens, read
        // transposed in bf16 and converted to fp16
        const u16* vbase = tile + (4 * q4 + (r16 >> 2)) * STRIDE + (G + j) * DH + 4 * (r16 & 3);
#pragma unroll
        for (int n = 0; n < DH / 16; ++n) {
            const u32x2 lo = lds_read_tr16(vbase + 16 * n);
            if constexpr (TR == 16) {
                const f16x4 a = __builtin_bit_cast(f16x4, u32x2{bf2_to_h2(lo[0]), bf2_to_h2(lo[1])});
#pragma unroll
                for (int rg = 0; rg < RPW; ++rg)
                    oacc[rg][n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pb4[rg], oacc[rg][n], 0, 0, 0);
            } else {
                const u32x2 hi = lds_read_tr16(vbase + 16 * n + 16 * STRIDE);
                const f16x8 a = as_f16x8(u32x4{bf2_to_h2(lo[0]), bf2_to_h2(lo[1]), bf2_to_h2(hi[0]), bf2_to_h2(hi[1])});
#pragma unroll
                for (int rg = 0; rg < RPW; ++rg) oacc[rg][n] = mfma16h(a, pb8[rg], oacc[rg][n]);
            }
        }
    }

#pragma unroll
    for (int rg = 0; rg < RPW; ++rg) {
        if (!row_ok[rg]) continue;
        const float l = wave_sum16x4(st[rg].l);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const size_t prow = (size_t)p * batch * s_q * h_q + qrow[rg];
        float* po = part_o + prow * DH;
#pragma unroll
        for (int n = 0; n < DH / 16; ++n) *reinterpret_cast<floatx4*>(po + 16 * n + 4 * q4) = oacc[rg][n] * inv;
        if (q4 == 0) part_lse[prow] = l > 0.f ? (st[rg].m + __log2f(l)) * kLn2 : kNegInf;
    }
}

template <int G, int NW, int RPW, int TR>
hipError_t launch_gqa_dma_t(const DecodeArgs& a, hipStream_t st) {
    const int rows_g = a.s_q * (a.h_q / a.g);
    const int waves = G * ((rows_g + 15) / 16) / RPW;
    const int nz = (waves + NW - 1) / NW;
    const int units = a.n_split * a.batch;
    // work items that run at once
    static const int per_cu = blocks_per_cu(gqa_dma_kernel<G, NW, RPW, TR>, NW * 64);
    const int cap = per_cu * a.cus / nz;
    dim3 grid(((units + 7) / 8) * 8 * nz);
    hipError_t e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gqa_dma_kernel<G, NW, RPW, TR>), grid, dim3(NW * 64), 0, st,
                       (const u16*)a.q_nope, (const u16*)a.q_rope, (const u16*)a.cache, a.bstride,
                       a.ctx_lens, a.max_ctx, a.h_q, a.s_q, a.chunk, a.n_split, nz, cap, a.batch, a.scale * kLog2e,
                       a.part_o, a.part_lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

template <int G, int NW, int RPW, int AHEAD>
hipError_t launch_gqa_t(const DecodeArgs& a, hipStream_t st) {
    const int rows_g = a.s_q * (a.h_q / a.g);
    const int waves = G * ((rows_g + 15) / 16) / RPW;
    const int nz = (waves + NW - 1) / NW;
    const int units = a.n_split * a.batch;
    // work items that run at once
    static const int per_cu = blocks_per_cu(gqa_decode_kernel<G, NW, RPW, AHEAD>, NW * 64);
    const int cap = per_cu * a.cus / nz;
    dim3 grid(((units + 7) / 8) * 8 * nz);
    hipError_t e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gqa_decode_kernel<G, NW, RPW, AHEAD>), grid, dim3(NW * 64), 0, st,
                       (const u16*)a.q_nope, (const u16*)a.q_rope, (const u16*)a.cache, a.bstride,
                       a.ctx_lens, a.max_ctx, a.h_q, a.s_q, a.chunk, a.n_split, nz, cap, a.batch, a.scale * kLog2e,
                       a.part_o, a.part_lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

// 8 waves per block (with 1024-thread blocks the 128-register cap spills the staging
// registers).  Two row tiles per wave when a group has an even number of them and one
// tile per wave would take more than one block.  Which kernel, as measured on MI355X
// (kernel time, HBM fraction of 8 TB/s):
//   - two row tiles per wave: direct loads (g = 8, s_q = 2, ragged 1K-32K: 0.777 ->
//     0.816 against register-staged 16-row tiles; g = 4, s_q = 2: 0.695 -> 0.731), but
//     at g = 1 (640-byte rows: a 32-row tile is 20 KB, too little in flight per block);
//   - one row tile per wave at g = 2 and 4: direct loads (g = 2: 0.62-0.66 -> 0.69-0.76;
//     g = 4: within 3 % either way at 4096-token chunks, 0.75 -> 0.77 at 1024);
//   - one row tile per wave at g = 8: register-staged 32-row tiles (0.860 against 0.852
//     at 4096-token chunks) except for chunks of at most 1024 tokens (0.800 -> 0.822);
//   - g = 1: register-staged, two 32-row tiles ahead.
template <int G>
hipError_t launch_gqa_g(const DecodeArgs& a, hipStream_t st) {
    const int rt = (a.s_q * (a.h_q / a.g) + 15) / 16;
    const bool two = rt % 2 == 0 && G * rt > 8;
    if constexpr (G == 1) {
        return two ? launch_gqa_t<1, 8, 2, 1>(a, st) : launch_gqa_t<1, 8, 1, 2>(a, st);
    } else if constexpr (G == 8) {
        if (two) return launch_gqa_dma_t<8, 8, 2, 16>(a, st);
        if (a.chunk <= 1024) return launch_gqa_dma_t<8, 8, 1, 16>(a, st);
        return launch_gqa_t<8, 8, 1, 1>(a, st);
    } else {
        return two ? launch_gqa_dma_t<G, 8, 2, 32>(a, st) : launch_gqa_dma_t<G, 8, 1, 32>(a, st);
    }
}

}  // namespace

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

}  // namespace gqla
