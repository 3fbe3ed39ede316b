// bf16 MFMA absorb decode for gfx950: the absorbed-query prologue and the latent
// attention kernel with the W_UV up-projection fused into its epilogue.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Architecture, MQA-absorb path).  Head i
// of group j = i / (h_q/g) attends over the shared latent rows [c_t | k_R,t]:
//   q~ = W_UK[j]^T q^N,  score_t = scale ([q~ | q^R].[c_t | k_R,t]),
//   u = sum_t softmax(score)_t c_t,  o = W_UV[j] u,
// over the visible tokens t <= L_b - s_q + s of query token s, one context chunk per
// workgroup (split-K).  With one chunk per sequence the workgroup writes o and the
// log-sum-exp itself; otherwise it writes the chunk's partials and launch_combine
// merges them.
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

constexpr int DH = 128;   // per-group value width
constexpr int DR = 64;    // rotary key width
constexpr int RK = 512;   // latent width
constexpr int W = RK + DR;
constexpr int TT = 32;    // tokens per tile

// Absorbed-query records, written by the prologue and read once by the attention
// kernel, QREC bytes per query row.  Per row they hold
//   hi: bf16 of x = q~ * scale * log2(e) (512 elements),
//   lo: bf16 of x - hi (the rounding residual of hi, rounded again) (512),
//   q^R (bf16, as given, unscaled) (64),
// stored for each 16 consecutive query rows (b * s_q * h_q + rho, rho = 16 m .. 16 m + 15)
// as one block of 34 pieces of 1 KB, in the order the score wave of those rows loads them:
// piece kk (hi, kk = 0..15), 16 + kk (lo) or 32 + kr (q^R, kr = 0..1) holds, at byte
// 16 (16 q + r) (lane (q, r) of the wave), elements 32 kk + 8 q .. + 7 of row r.  Each
// load instruction then reads 1 KB of contiguous memory; the rows themselves, 16 rows x
// 64 bytes per instruction, load at well under that rate.  (rec_piece gives the offset.)
// hi + lo carries x to about 16 significant bits, against the bf16 latent rows as they
// are stored (every product exact in the fp32 accumulation).  A single 8- or 11-bit
// rounding of q~ gives score errors that grow with |score|: with sharp softmaxes (peak
// logits of 30-40 in log2 units) they alone exceed the 2e-3 + 2e-2 |o| bound several-
// fold; the hi + lo pair leaves them far below it, at one extra MFMA per latent k-step.
// bf16 keeps fp32's exponent range, so no operand of the score product needs scaling.
constexpr int QREC = 2176;
constexpr int QHI = 0, QLO = 16, QROPE = 32;   // first piece of each part

// Byte offset of piece m of query row `row`'s 16-row block, lane (q, r) position for r =
// row % 16 (the caller adds nothing else).
__device__ __forceinline__ size_t rec_piece(size_t row, int m, int q) {
    return (row / 16) * (16 * (size_t)QREC) + (size_t)m * 1024 + (size_t)(q * 16 + (int)(row % 16)) * 16;
}

// ---------------------------------------------------------------------------
// Prologue: one block per (64 rows of group j, j, quarter qc of the latent columns); 4
// waves of 16 rows.  Rows of group j are numbered iota = (b*s_q + s)*hpg + hh.  The
// contraction runs over d, strided in the [g][d_h][r_kv] layout, so the block stages its
// quarter of W_UK[j]'s columns (128 d x 128 r, 36 KB with the pad) row-major in LDS and
// forms the A operand (W_UK^T) with transposing LDS reads: 4 rows d x 16 columns r per
// 16-lane group.  A lane ends with the 32 columns 128 qc + 16 mt + 4 q4 + i (mt = 0..7,
// i = 0..3) of its row r16.  Four blocks per row block keep even small batches on more
// compute units than one block per row block would (one per 64 rows and group).
// ---------------------------------------------------------------------------
constexpr int PRO_COLS = RK / 4;
constexpr int PRO_STRIDE = PRO_COLS + 16;

// W_UV in the order the attention kernel's epilogue reads it: for group j, 128-column
// block cb, 16-row tile dt and k-step ks, the 64 lanes' 16-byte A operands (lane (q, r16):
// row 16 dt + r16, columns 128 cb + 32 ks + 8 q .. + 7) lie side by side, so one wave
// instruction loads 1 KB of contiguous memory (the rows of W_UV itself give 64 bytes per
// row and 16 rows per instruction, at well under half the rate).  Element offset (u16).
__device__ __forceinline__ size_t wpack_index(int j, int cb, int dt, int ks, int lane) {
    return ((((size_t)j * 4 + cb) * (DH / 16) + dt) * 4 + ks) * 512 + (size_t)lane * 8;
}

__global__ __launch_bounds__(256) void absorb_prologue_kernel(
    const u16* __restrict__ q_nope, const u16* __restrict__ q_rope, const u16* __restrict__ w_uk,
    const u16* __restrict__ w_uv, unsigned char* __restrict__ qrec, u16* __restrict__ wpack, int batch, int h_q,
    int g, int s_q, float scale_log2) {
    __shared__ __attribute__((aligned(16))) u16 wt[DH * PRO_STRIDE];
    const int j = blockIdx.y, qc = blockIdx.z;
    const int tid = threadIdx.x;
    // W_UV[j], columns 128 qc .. 128 qc + 127, in the attention kernel's epilogue operand
    // order (see wpack_index): eight 16-row tiles dt of 256 pieces of 16 bytes, one piece
    // per thread.  The first min(8, row blocks) row blocks share the tiles out; the first
    // tile of each is loaded beside the W_UK staging below.
    const int nwb = min((int)gridDim.x, DH / 16);
    const bool wrep = blockIdx.x < nwb;
    const int wln = tid & 63, wks = tid >> 6;
    auto wsrc = [&](int dt) {
        return reinterpret_cast<const u32x4*>(w_uv + ((size_t)j * DH + 16 * dt + (wln & 15)) * RK + PRO_COLS * qc +
                                              32 * wks + 8 * (wln >> 4));
    };
    auto wdst = [&](int dt) { return reinterpret_cast<u32x4*>(wpack + wpack_index(j, qc, dt, wks, wln)); };
    u32x4 wv = {0u, 0u, 0u, 0u};
    if (wrep) wv = *wsrc(blockIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;

    // stage columns 128 qc .. 128 qc + 127 of W_UK[j]: 2048 chunks of 16 bytes, 8 per
    // thread, all eight loads in flight before the first store
    constexpr int CPRW = PRO_COLS / 8;   // 16-byte chunks per staged row
    {
        const u16* wj = w_uk + (size_t)j * DH * RK + qc * PRO_COLS;
        u32x4 v[DH * CPRW / 256];
#pragma unroll
        for (int k = 0; k < DH * CPRW / 256; ++k) {
            const int c = k * 256 + tid;
            v[k] = *reinterpret_cast<const u32x4*>(wj + (size_t)(c / CPRW) * RK + (c % CPRW) * 8);
        }
#pragma unroll
        for (int k = 0; k < DH * CPRW / 256; ++k) {
            const int c = k * 256 + tid;
            *reinterpret_cast<u32x4*>(wt + (c / CPRW) * PRO_STRIDE + (c % CPRW) * 8) = v[k];
        }
    }
    if (wrep) {
        *wdst(blockIdx.x) = wv;
        // grids of fewer than eight row blocks: the remaining tiles
        for (int dt = blockIdx.x + nwb; dt < DH / 16; dt += nwb) *wdst(dt) = *wsrc(dt);
    }

    const int hpg = h_q / g;
    const int nrows = batch * s_q * hpg;
    const int iota = blockIdx.x * 64 + wave * 16 + r16;
    const bool ok = iota < nrows;
    const int bs = ok ? iota / hpg : 0;
    const int hh = ok ? iota - bs * hpg : 0;
    const int b = bs / s_q, s = bs - (bs / s_q) * s_q;
    const int h = j * hpg + hh;
    const size_t qrow = ((size_t)b * s_q + s) * h_q + h;

    // k-slot e of lane group q4 in k-step kd is d = 32kd + 4q4 + e (e < 4) or
    // 32kd + 16 + 4q4 + (e - 4): the transposing reads of the four lane groups then lie
    // 4 rows apart, 32 banks at this row stride, so they do not conflict
    bf16x8 qb[DH / 32];
#pragma unroll
    for (int kd = 0; kd < DH / 32; ++kd) {
        if (ok) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(q_nope + qrow * DH + kd * 32 + q4 * 4);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(q_nope + qrow * DH + kd * 32 + 16 + q4 * 4);
            qb[kd] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        } else {
            qb[kd] = zero_bf16x8();
        }
    }
    __syncthreads();

    floatx4 acc[PRO_COLS / 16];
    const u16* abase = wt + (4 * q4 + (r16 >> 2)) * PRO_STRIDE + 4 * (r16 & 3);
#pragma unroll
    for (int mt = 0; mt < PRO_COLS / 16; ++mt) {
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kd = 0; kd < DH / 32; ++kd) {
            const u16* pa = abase + kd * 32 * PRO_STRIDE + mt * 16;
            const u32x2 lo = lds_read_tr16(pa);
            const u32x2 hi = lds_read_tr16(pa + 16 * PRO_STRIDE);
            a = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), qb[kd], a);
        }
        acc[mt] = a;
    }

    // x = q~ * scale * log2(e) (fp32) as hi = bf16(x) and lo = bf16(x - hi), staged in
    // LDS (over the W_UK tile, once every wave is done with it) as [row][hi 128 | lo 128]
    // so that the records leave in whole 256-byte segments: written straight from the
    // MFMA layout, every store instruction would touch 16 rows with 32 bytes each.
    constexpr int OSTR = 2 * PRO_COLS + 8;   // staged row stride (u16): 132 dwords
    static_assert(64 * OSTR <= DH * PRO_STRIDE, "the staged records fit over the W_UK tile");
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < PRO_COLS / 16; ++mt) {
        u16 hs[4], ls[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = acc[mt][i] * scale_log2;
            hs[i] = f2bf(x);
            ls[i] = f2bf(x - bf2f(hs[i]));
        }
        u16* srow = wt + (wave * 16 + r16) * OSTR + 16 * mt + 4 * q4;
        *reinterpret_cast<u32x2*>(srow) = u32x2{pack2(hs[0], hs[1]), pack2(hs[2], hs[3])};
        *reinterpret_cast<u32x2*>(srow + PRO_COLS) = u32x2{pack2(ls[0], ls[1]), pack2(ls[2], ls[3])};
    }
    __syncthreads();
    // query row of block row r, and whether it exists
    auto row_of = [&](int r, bool& valid) -> size_t {
        const int it = blockIdx.x * 64 + r;
        valid = it < nrows;
        const int bs_ = valid ? it / hpg : 0;
        const int hh_ = valid ? it - bs_ * hpg : 0;
        const int b_ = bs_ / s_q, s_ = bs_ - (bs_ / s_q) * s_q;
        return ((size_t)b_ * s_q + s_) * h_q + j * hpg + hh_;
    };
    // 64 rows x 32 pieces of 16 bytes (16 of hi, 16 of lo), in units of one piece m of
    // 16 consecutive block rows: unit u = 4 k + wave is rows 16 (u / 8) + r, piece
    // (u % 8 < 4 ? hi : lo) k-step 4 qc + u % 4, lane (q, r).  Where those rows are 16
    // consecutive query rows (h_q / g >= 16), a wave instruction writes one whole 1 KB
    // piece of their record block.
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int u = k * 4 + wave;
        const int r = 16 * (u >> 3) + r16, mi = u & 7;
        bool valid;
        const size_t row = row_of(r, valid);
        if (valid) {
            const int c = (mi < 4 ? 0 : 16) + 4 * (mi & 3) + q4;   // staged piece: 8 columns
            const u32x4 v = *reinterpret_cast<const u32x4*>(wt + r * OSTR + c * 8);
            *reinterpret_cast<u32x4*>(qrec + rec_piece(row, (mi < 4 ? QHI : QLO) + 4 * qc + (mi & 3), q4)) = v;
        }
    }
    // q^R: 64 elements (8 pieces of 16 bytes) per row, copied by the first quarter's block,
    // in the same units (u = 4 k + wave: rows 16 (u / 2) + r, piece kr = u % 2)
    if (qc == 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int u = k * 4 + wave;
            const int r = 16 * (u >> 1) + r16, kr = u & 1;
            bool valid;
            const size_t qr = row_of(r, valid);
            if (valid)
                *reinterpret_cast<u32x4*>(qrec + rec_piece(qr, QROPE + kr, q4)) =
                    *reinterpret_cast<const u32x4*>(q_rope + qr * DR + kr * 32 + q4 * 8);
        }
    }
}

// ---------------------------------------------------------------------------
// Latent attention: absorb_decode_kernel<NS>.
//
// Work split.  A workgroup takes one (context chunk, sequence) pair and R = 16 NS of the
// s_q*h_q query rows.  Its waves are specialised:
//   - NS score waves: score wave s owns rows 16 s .. 16 s + 15 of the block and the
//     whole tile's 32 tokens.  It holds that row tile's absorbed queries in registers
//     (hi, lo and rotary parts: 136 VGPRs), computes
//       S^T[token][row] = C_tile . q^T   (A = latent rows from LDS, B = queries)
//     on the 16x16x32 bf16 MFMA, keeps the online softmax state of its rows and writes
//     P (fp16, in the B-operand layout of the value MFMA) and each row's rescale
//     factor to LDS.
//   - 4 value waves: value wave v owns latent columns 128 v .. 128 v + 127 of u for all
//     R rows (u: 128 VGPRs at R = 64) and computes
//       U^T[col][row] += C_tile^T . P^T  (A = latent columns from LDS with the gfx950
//                                          transposing read, B = P from LDS)
//     on the 16x16x32 fp16 MFMA, converting its A operands from bf16 in registers.
//     Value waves also stream the tiles from HBM.
// Waves w and w + 4 share a SIMD, so at R = 64 each SIMD runs one score and one value
// wave.  Score waves issue at a raised priority: their MFMAs go first, and the value
// wave's operand conversion (VALU) runs beside them; the value wave's MFMAs follow,
// beside the score wave's softmax.  Splitting u
// by columns over value waves and q by rows over score waves keeps both within 256
// registers: u for 128 rows is 256 KB and q^ (hi + lo) 278 KB, more than a CU's 512 KB
// register file together, so a workgroup takes 64 rows and the 2 (s_q = 1) or 4
// (s_q = 2) row blocks of a (chunk, sequence) pair run as workgroups 8 ids apart, on one
// XCD, where the second read of every tile is an L2 hit.
//
// Pipeline.  Tiles (32 rows x 576 bf16, one contiguous span of HBM) go straight from
// global memory into LDS with global_load_lds_dwordx4 (lane l of a wave instruction
// lands at base + 16 l), into four buffers, and are used there as loaded: nothing is
// written to a tile buffer but the loads themselves (LDS writes run at well under half
// the read rate on gfx950, so a conversion pass through LDS would cost as much as all
// the operand reads).  At step k, after the barrier that published tile k:
//   score waves:  scores and softmax of tile k (buffer k%4), P and rescale factors to
//                 the P buffer k%2;
//   value waves:  issue the loads of tile k+2 (buffer (k+2)%4, last read at step k-1),
//                 then U += C_{k-1}^T P_{k-1} (buffer (k-1)%4, P buffer (k-1)%2), then
//                 wait until their own loads of tile k+1 (issued at step k-1) have landed;
// then one barrier.  LDS: 4 tiles of 32 x (576 + 16) bf16 (148 KB) + 2 P buffers.  Rows
// past the chunk are loaded as copies of the tile's first row (finite data, P = 0).
// The row stride of 576 + 16 elements (8 x odd dwords modulo the 64 banks) keeps both
// the 16-byte operand reads of 16 rows and the transposing reads of 4 rows x 32 bytes
// free of bank conflicts (measured at the full LDS read rate on gfx950).
//
// Scores.  x = hi + lo against the tile's bf16 latent accumulates the latent part of the
// log2-domain logit; the rotary part multiplies q^R and k_R as given and is scaled after
// the MFMA: s = acc + scale log2(e) accr.
//
// Softmax.  Online, with a lazily raised reference: exponentials are taken against a
// per-row reference m (log2 domain) raised only when a tile's maximum exceeds it by more
// than kLazy, so p = 2^(s - m) <= 2^kLazy, which fp16 P and fp32 sums hold as precisely as
// values <= 1.  P is fp16 rather than bf16: its 11-bit significand keeps the weights'
// rounding well inside the bound, where bf16's 8 bits would exceed it on sharp softmaxes.  When a row that has accumulated raises its reference, the value waves
// multiply its u columns by alpha = 2^(m_old - m_new) before adding the tile; the score
// wave writes alpha (1 otherwise) beside P.  Normalisation and log-sum-exp use the same
// reference, so the result is the exact softmax's.
//
// Epilogue.  u / l is split into three bf16 terms (about 24 significant bits); each
// value wave multiplies its 128 columns by the matching columns of W_UV[j] on the bf16
// MFMA (a partial sum over those columns), the four partials meet in LDS, and every
// wave sums and writes a share of the block's R x 128 outputs.
//
// Grid.  One-dimensional and XCD-aware: blocks with ids 8 apart run on one XCD.
// ---------------------------------------------------------------------------
constexpr float kLazy = 10.f;
constexpr int STRIDE = W + 16;                 // LDS row stride in elements
constexpr int SROW = STRIDE / 8;               // 16-byte slots per LDS row (72 data + 2 pad)
constexpr int CPR = W / 8;                     // data slots per row
constexpr int TSLOTS = TT * SROW;              // slots of a tile buffer
constexpr int NINST = (TSLOTS + 63) / 64;      // 64-lane load instructions per tile (37)
constexpr int NV = 4;                          // value waves
constexpr int VI = (NINST + NV - 1) / NV;      // load instructions per value wave (<= 10)
constexpr int VCOLS = RK / NV;                 // latent columns of u per value wave (128)
constexpr int NCT = VCOLS / 16;                // 16-wide column tiles per value wave (8)

struct SoftmaxState {
    float m;   // reference (log2 domain), identical in the 4 lanes of a row; -inf before any score
    float l;   // lane-partial running sum of 2^(s - m)
};

// sc[e]: log2-domain scores of the lane's 8 tokens (masked: -inf).  Returns P as the fp16
// B operand.  need: this row has accumulated under its old reference and raised it, so
// its accumulators must be multiplied by alpha before this tile's P is added.
__device__ __forceinline__ f16x8 softmax_tile(SoftmaxState& st, const float (&sc)[8], bool& need, float& alpha) {
    float mt = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mt = wave_max16x4(mt);
    const bool raise = mt > st.m + kLazy;   // false while the row has seen nothing but -inf
    need = raise && st.m != kNegInf;        // a fresh row's accumulators are still zero
    alpha = raise ? fast_exp2(st.m - mt) : 1.f;
    st.l *= alpha;
    st.m = raise ? mt : st.m;
    const float muse = (st.m == kNegInf) ? 0.f : st.m;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(sc[e] - muse);
    st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    return as_f16x8(u32x4{pack2h(p[0], p[1]), pack2h(p[2], p[3]), pack2h(p[4], p[5]), pack2h(p[6], p[7])});
}

template <int NS>
__global__ __launch_bounds__((NS + NV) * 64) void absorb_decode_kernel(
    const unsigned char* __restrict__ qrec, const u16* __restrict__ wpack, const u16* __restrict__ cache,
    int64_t bstride, const int32_t* __restrict__ ctx_lens, int max_ctx, int h_q, int g, int s_q, int chunk,
    int n_split, int nz, int cap, int batch, float scale_log2, float* __restrict__ part_o, float* __restrict__ part_lse,
    u16* __restrict__ out, float* __restrict__ lse_out) {
    constexpr int R = 16 * NS;                     // query rows of a workgroup
    static_assert(NS >= 1 && NS <= 4, "1..4 score waves");
    static_assert(NS * 8 * 64 * 16 <= TSLOTS * 16, "a value wave's epilogue partials fit in one tile buffer");
    // One block of LDS with the small, often-addressed arrays first: ds_read/ds_write
    // carry a 16-bit immediate offset, so everything below 64 KB is reached from one
    // per-lane base register; the tile buffers above it need a base per buffer.
    struct Lds {
        u16 pbuf[2][NS * 64 * 8];                  // P of the last two tiles (B-operand layout)
        float abuf[2][R];                          // per-row rescale factor of each P buffer
        float lfin[R], mfin[R];                    // final softmax sum and reference per row
        u16 tiles[4][TSLOTS * 8];                  // tile buffers, tile k in buffer k % 4
    };
    __shared__ __attribute__((aligned(16))) Lds lds;
    auto& pbuf = lds.pbuf;
    auto& abuf = lds.abuf;
    auto& lfin = lds.lfin;
    auto& mfin = lds.mfin;

    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int z = slot % nz;
    const int pair = (slot / nz) * 8 + xcd;
    if (pair >= n_split * batch) return;           // padding of the last group of 8
    // One chunk per sequence: item k is sequence k.  Several: the items are ordered
    // longest first (chunk_of_item), so the short last chunks of a ragged batch fill in
    // at the end.
    int b = pair, p = 0, t0 = 0, t1 = 0;
    if (n_split > 1) {
        if (!chunk_of_item<(NS + NV) * 64>(pair, ctx_lens, batch, max_ctx, chunk, cap,
                                           reinterpret_cast<int*>(lds.tiles[0]), b, p, t0, t1))
            return;
        __syncthreads();   // the item is known to every thread before the tiles reuse LDS
    }
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    if (n_split == 1) t1 = min(chunk, L);
    const int RQ = s_q * h_q;
    const int na = min(NS, (RQ - z * R) / 16);     // active row tiles of the block (RQ % 16 == 0)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q4 = lane >> 4, r16 = lane & 15;
    const bool direct = n_split == 1;

    if (t0 >= L) {
        // nothing visible in this chunk; with one chunk per sequence the block writes the
        // empty result (o = 0, lse = -inf) itself
        if (direct) {
            for (int e = tid; e < na * 16 * (DH / 8); e += (NS + NV) * 64) {
                const int rho = z * R + e / (DH / 8);
                const int s = rho / h_q, h = rho - (rho / h_q) * h_q;
                *reinterpret_cast<u32x4*>(out + (((size_t)b * s_q + s) * h_q + h) * DH + (e % (DH / 8)) * 8) =
                    u32x4{0u, 0u, 0u, 0u};
                if (lse_out && e % (DH / 8) == 0) lse_out[((size_t)b * s_q + s) * h_q + h] = kNegInf;
            }
        }
        return;
    }
    const int ntiles = (t1 - t0 + TT - 1) / TT;
    // tokens below t_full are visible to every query row and inside the chunk
    const int t_full = min(t1, clampi(L - s_q + 1, 0, L));

    const u16* seq = cache + (size_t)b * bstride + (size_t)t0 * W;

    auto bufp = [&](int i) -> u16* { return lds.tiles[i & 3]; };   // buffer of tile i

    // The two roles run separate code with the same sequence of barriers (one before the
    // tile loop, one per step, one in the epilogue), so that the compiler
    // never holds the score waves' queries and the value waves' accumulators at once.
    if (wave < NS) {
        // ============================== score wave: row tile sw
        // Its MFMAs go first on the SIMD; the value wave's MFMAs fill in behind them,
        // mostly while this wave runs its softmax.
        __builtin_amdgcn_s_setprio(1);
        const int sw = wave;
        const bool active = sw < na;
        bf16x8 qhi[RK / 32], qlo[RK / 32], qro[DR / 32];
        int nvis = 0;
        SoftmaxState st{kNegInf, 0.f};
        if (active) {
            const int rho = z * R + 16 * sw + r16;
            // this row tile's block of records (16 rows; RQ is a multiple of 16)
            const unsigned char* blk = qrec + ((size_t)b * RQ + z * R + 16 * sw) / 16 * (16 * (size_t)QREC) + lane * 16;
#pragma unroll
            for (int kk = 0; kk < RK / 32; ++kk) {
                qhi[kk] = ld_bf16x8(reinterpret_cast<const u16*>(blk + (QHI + kk) * 1024));
                qlo[kk] = ld_bf16x8(reinterpret_cast<const u16*>(blk + (QLO + kk) * 1024));
            }
#pragma unroll
            for (int kr = 0; kr < DR / 32; ++kr) qro[kr] = ld_bf16x8(reinterpret_cast<const u16*>(blk + (QROPE + kr) * 1024));
            nvis = clampi(L - s_q + rho / h_q + 1, 0, L);
        }
        auto sstep = [&](int k) {
            if (active && k < ntiles) {
                const u16* const tile = bufp(k);
                u16* const pw = pbuf[k & 1];
                float* const aw = abuf[k & 1];
                const int tb = t0 + k * TT;
                floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, accr0 = acc0, accr1 = acc0;
                const u16* arow = tile + r16 * STRIDE + q4 * 8;
                // k-step j = 0..17 reads columns 32 j .. 32 j + 31 (latent for j < 16, rotary
                // after); its operand reads are issued PF steps ahead of its MFMAs, which the
                // scheduling barriers keep in this order
                constexpr int KS = W / 32, PF = 6;
                bf16x8 ra0[PF + 1], ra1[PF + 1];
#pragma unroll
                for (int j = 0; j < PF; ++j) {
                    ra0[j] = ld_bf16x8(arow + j * 32);
                    ra1[j] = ld_bf16x8(arow + 16 * STRIDE + j * 32);
                }
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    if (j + PF < KS) {
                        ra0[(j + PF) % (PF + 1)] = ld_bf16x8(arow + (j + PF) * 32);
                        ra1[(j + PF) % (PF + 1)] = ld_bf16x8(arow + 16 * STRIDE + (j + PF) * 32);
                    }
                    const bf16x8 a0 = ra0[j % (PF + 1)], a1 = ra1[j % (PF + 1)];
                    if (j < RK / 32) {
                        acc0 = mfma16(a0, qhi[j], acc0);
                        acc1 = mfma16(a1, qhi[j], acc1);
                        acc0 = mfma16(a0, qlo[j], acc0);
                        acc1 = mfma16(a1, qlo[j], acc1);
                    } else {
                        accr0 = mfma16(a0, qro[j - RK / 32], accr0);
                        accr1 = mfma16(a1, qro[j - RK / 32], accr1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                float sc[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sc[i] = fmaf(accr0[i], scale_log2, acc0[i]);
                    sc[4 + i] = fmaf(accr1[i], scale_log2, acc1[i]);
                }
                if (tb + TT > t_full) {
#pragma unroll
                    for (int th = 0; th < 2; ++th)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int t = tb + th * 16 + q4 * 4 + i;
                            if (!(t < t1 && t < nvis)) sc[th * 4 + i] = kNegInf;
                        }
                }
                bool need;
                float alpha;
                const f16x8 pb = softmax_tile(st, sc, need, alpha);
                *reinterpret_cast<u32x4*>(pw + (sw * 64 + lane) * 8) = __builtin_bit_cast(u32x4, pb);
                if (q4 == 0) aw[16 * sw + r16] = need ? alpha : 1.f;
                if (k == ntiles - 1) {
                    const float l = wave_sum16x4(st.l);
                    if (q4 == 0) {
                        lfin[16 * sw + r16] = l;
                        mfin[16 * sw + r16] = st.m;
                    }
                }
            }
            block_sync();
        };
        if (!active) {
            // a row tile past s_q*h_q: P = 0 and rescale factor 1 in both P buffers, so the
            // value waves' loop needs no per-tile condition; final sum 0
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                *reinterpret_cast<u32x4*>(pbuf[j] + (sw * 64 + lane) * 8) = u32x4{0u, 0u, 0u, 0u};
                if (q4 == 0) abuf[j][16 * sw + r16] = 1.f;
            }
            if (q4 == 0) {
                lfin[16 * sw + r16] = 0.f;
                mfin[16 * sw + r16] = kNegInf;
            }
        }
        block_sync();   // tile 0 converted
#pragma unroll 1
        for (int k = 0; k <= ntiles; ++k) sstep(k);
        if (active && q4 == 0) {
            const int rho = z * R + 16 * sw + r16;
            const int s = rho / h_q, h = rho - (rho / h_q) * h_q;
            const float l = lfin[16 * sw + r16];
            const float v = l > 0.f ? (mfin[16 * sw + r16] + __log2f(l)) * kLn2 : kNegInf;
            if (direct) {
                if (lse_out) lse_out[((size_t)b * s_q + s) * h_q + h] = v;
            } else {
                part_lse[((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h] = v;
            }
        }
    } else {
        // ============================== value wave: latent columns VCOLS vw .. + VCOLS - 1
        const int vw = wave - NS;
        floatx4 uacc[NCT][NS];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int rt = 0; rt < NS; ++rt) uacc[ct][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
        // Byte offset within a tile of the chunk that each of this lane's load slots carries,
        // two 16-bit offsets per register (a tile is 36,864 bytes).  The 37 instructions of a
        // tile cover its 2368 slots exactly; the two pad slots of an LDS row load that row's
        // first 16 bytes (a line the row's first slot loads anyway) and are never read, so
        // every instruction loads all 64 lanes without a condition.
        static_assert(NINST * 64 == TSLOTS, "load instructions cover the tile exactly");
        uint32_t dma_off2[(VI + 1) / 2];
#pragma unroll
        for (int i = 0; i < (VI + 1) / 2; ++i) dma_off2[i] = 0;
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const int sl = (vw + NV * i) * 64 + lane;
            const int r = sl / SROW, c = sl - (sl / SROW) * SROW;
            const uint32_t o = sl < TSLOTS ? (uint32_t)((r * W + (c < CPR ? c : 0) * 8) * 2) : 0u;
            dma_off2[i / 2] |= o << (16 * (i & 1));
        }
        auto slot_off = [&](int i) -> uint32_t { return (dma_off2[i / 2] >> (16 * (i & 1))) & 0xffffu; };
        // The offsets are loop-invariant; left visible, the compiler unpacks (and for the
        // tail, reduces) all of them before the tile loop and runs out of registers.
        // Re-declaring them opaque at each step keeps them packed.
        auto opaque_offsets = [&]() {
#pragma unroll
            for (int i = 0; i < (VI + 1) / 2; ++i) asm volatile("" : "+v"(dma_off2[i]));
        };
        const bool full = vw < NINST % NV || NINST % NV == 0;   // this wave issues VI loads per tile (else VI - 1)
        // Instruction i of value wave vw fills slots (vw + 4 i) * 64 .. + 63 of a tile buffer.
        auto dma_one = [&](const u16* tsrc, uint32_t off, uint32_t tbuf, int i) {
            if (i < VI - 1 || full) dma16(tsrc, off, tbuf + (uint32_t)((vw + NV * i) * 1024));
        };
        // All loads of tile `it` at once; rows past the chunk load the tile's first row.
        auto dma_tile = [&](int it, uint32_t tbuf) {
            const u16* tsrc = seq + (size_t)it * TT * W;
            const int rows = t1 - t0 - it * TT;
            if (rows >= TT) {
#pragma unroll
                for (int i = 0; i < VI; ++i) dma_one(tsrc, slot_off(i), tbuf, i);
            } else {
                const uint32_t lim = (uint32_t)(rows * W * 2);
#pragma unroll
                for (int i = 0; i < VI; ++i) {
                    const uint32_t o = slot_off(i);
                    dma_one(tsrc, o < lim ? o : o % (uint32_t)(W * 2), tbuf, i);
                }
            }
        };
        // wait until this wave's loads of the older tile have landed, leaving the loads of
        // the newer tile (issued after them, when `newer`) in flight
        auto wait_own = [&](bool newer) {
            if (!newer) {
                wait_vmcnt<0>();
            } else if (full) {
                wait_vmcnt<VI>();
            } else {
                wait_vmcnt<VI - 1>();
            }
        };
        // lane offset of the transposing reads of column tile 0 of this wave's columns
        const int goff = (4 * q4 + (r16 >> 2)) * STRIDE + VCOLS * vw + 4 * (r16 & 3);
        // Step k >= 1 of the pipeline: U += C_{k-1}^T P_{k-1}, loads of tile k+2, wait for
        // this wave's loads of tile k+1.
        // A operands of a step, all eight column tiles (transposing reads of bf16), read at
        // the end of the step before: after the barrier only P and the rescale factors
        // are left to read, and the barrier's burst of LDS requests is smaller
        u32x4 ra[NCT];
        auto read_a = [&](const u16* bt, int go) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const u16* p0 = bt + go + 16 * ct;
                const u32x2 lo = lds_read_tr16(p0);
                const u32x2 hi = lds_read_tr16(p0 + 16 * STRIDE);
                ra[ct] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        };
        auto vstep = [&](int k) {
            opaque_offsets();
            // per-lane bases, opaque per step: the addresses derived from them are then
            // recomputed in each step (one add each) instead of being hoisted out of the
            // loop for all four buffers and held in registers
            int go = goff, ln = lane;
            asm volatile("" : "+v"(go), "+v"(ln));
            const u16* const pr = pbuf[(k + 1) & 1];
            const float* const ar = abuf[(k + 1) & 1];
            const bool more = k + 2 < ntiles;
            // the loads of tile k+2 go out first: they have until the end of step k+1 to land
            if (more) dma_tile(k + 2, lds_addr(bufp(k + 2)));
            // The rescale factors and P are read (the A operands are already in flight
            // from the step before); the A operands are then converted to fp16, and only
            // after that do the MFMAs start: the conversion (VALU) runs beside the score
            // wave's MFMAs on this SIMD, and this wave's MFMAs beside the score wave's
            // softmax.
            float al[NS];
#pragma unroll
            for (int rt = 0; rt < NS; ++rt) al[rt] = ar[16 * rt + (ln & 15)];
            f16x8 pv[NS];
#pragma unroll
            for (int rt = 0; rt < NS; ++rt) pv[rt] = ld_f16x8(pr + (rt * 64 + ln) * 8);

            // rescale rows whose reference rose at tile k-1 (rare)
            bool any = false;
#pragma unroll
            for (int rt = 0; rt < NS; ++rt) any = any || al[rt] != 1.f;
            if (__builtin_expect(__any(any), 0)) {
                asm volatile("" ::: "memory");   // keeps the multiplies inside the branch
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int rt = 0; rt < NS; ++rt) uacc[ct][rt] *= al[rt];
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) ra[ct] = bf8_to_h8(ra[ct]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f16x8 a = as_f16x8(ra[ct]);
#pragma unroll
                for (int rt = 0; rt < NS; ++rt) uacc[ct][rt] = mfma16h(a, pv[rt], uacc[ct][rt]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (k < ntiles) read_a(bufp(k), go);   // the next step's A operands: tile k, in LDS since step k-1
            wait_own(more);
            block_sync();
        };
        // prologue of the pipeline: tiles 0 and 1 issued, tile 0 landed; then step 0 (loads
        // of tile 2, tile 1 landed)
        dma_tile(0, lds_addr(bufp(0)));
        const bool two = ntiles > 1;
        if (two) dma_tile(1, lds_addr(bufp(1)));
        wait_own(two);
        block_sync();
        {
            const bool more = 2 < ntiles;
            if (more) dma_tile(2, lds_addr(bufp(2)));
            wait_own(more);
            block_sync();
        }
        read_a(bufp(0), goff);
#pragma unroll 1
        for (int k = 1; k <= ntiles; ++k) vstep(k);
        // no direct load may still be writing this workgroup's LDS
        wait_vmcnt<0>();

        // u goes to tile buffer vw (free: the last step's barrier retired every tile), as
        // 8 KB per row tile.  Storing it at once ends the accumulators' lives at the loop
        // exit, so the epilogue never holds them next to its own registers.
        float* red = reinterpret_cast<float*>(bufp(vw));
#pragma unroll
        for (int rt = 0; rt < NS; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                *reinterpret_cast<floatx4*>(red + (((rt * 8) + ct) * 64 + lane) * 4) = uacc[ct][rt];
    }
    block_sync();   // u of every column block is in LDS

    // ---- epilogue: o^T = W_UV[j] (u / l)^T.  Unit (row tile rt, column block cb) is the
    // partial sum over latent columns VCOLS cb .. + VCOLS - 1 for the 16 rows of rt; the
    // units are dealt over all waves (score waves included), and each writes its partial
    // (8 KB) over the u it read.
    const int hpg = h_q / g;
#pragma unroll 1
    for (int un = wave; un < na * NV; un += NS + NV) {
        const int rt = un / NV, cb = un - (un / NV) * NV;
        float* blk = reinterpret_cast<float*>(bufp(cb)) + rt * 8 * 64 * 4;
        const float l = lfin[16 * rt + r16];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        // U^T as the B operand of o^T = W_UV[j] U^T: in k-step ks, k-slot e of lane group
        // q4 is latent column VCOLS cb + 32 ks + 8 q4 + e, so that each lane's weight
        // operand is 16 contiguous bytes of a W_UV row (read from the packed copy the
        // prologue wrote, where a wave's 64 operands are 1 KB in a row).  Column 16 ct + 4 q + i of u sits
        // in column tile ct, lane r16 + 16 q, element i of the stored accumulators, so
        // slots 0-3 come from lane group 2 (q4 & 1) and slots 4-7 from the next one, of
        // column tile 2 ks + q4 / 2.  u / l is carried as three bf16 terms (about 24
        // significant bits): o = W_UV u can cancel to values far below |u| (a one-hot
        // softmax over latent rows of magnitude 1e4 leaves u = c_t), and two terms
        // (16 bits) would then miss the 2e-3 absolute bound.
        bf16x8 ub[NCT / 2], um[NCT / 2], ul[NCT / 2];
        const int lq = r16 + 32 * (q4 & 1);
#pragma unroll
        for (int ks = 0; ks < NCT / 2; ++ks) {
            const int ctq = 2 * ks + (q4 >> 1);
            const floatx4 c0 = *reinterpret_cast<const floatx4*>(blk + (ctq * 64 + lq) * 4);
            const floatx4 c1 = *reinterpret_cast<const floatx4*>(blk + (ctq * 64 + lq + 16) * 4);
            u32x4 vh, vm, vl;
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
                const floatx4& src = (hh >> 1) ? c1 : c0;
                const float x = src[2 * (hh & 1)] * inv, y = src[2 * (hh & 1) + 1] * inv;
                const u16 xh = f2bf(x), yh = f2bf(y);
                const float xr = x - bf2f(xh), yr = y - bf2f(yh);
                const u16 xm = f2bf(xr), ym = f2bf(yr);
                vh[hh] = pack2(xh, yh);
                vm[hh] = pack2(xm, ym);
                vl[hh] = pack2f(xr - bf2f(xm), yr - bf2f(ym));
            }
            ub[ks] = as_bf16x8(vh);
            um[ks] = as_bf16x8(vm);
            ul[ks] = as_bf16x8(vl);
        }
        const int rho = z * R + 16 * rt + r16;
        const int jrow = (rho % h_q) / hpg;
        const int first = z * R + 16 * rt;
        const int jlo = (first % h_q) / hpg, jhi = ((first % h_q) + 15) / hpg;
        // each lane's row belongs to exactly one group jj of the row tile; its partial is
        // written in that group's pass
        for (int jj = jlo; jj <= jhi; ++jj) {
            // all of the group's weight operands for these columns are loaded before the
            // first MFMA (one round trip to L2 per unit and group)
            u32x4 wa[DH / 16][NCT / 2];
#pragma unroll
            for (int dt = 0; dt < DH / 16; ++dt)
#pragma unroll
                for (int ks = 0; ks < NCT / 2; ++ks)
                    wa[dt][ks] = *reinterpret_cast<const u32x4*>(wpack + wpack_index(jj, cb, dt, ks, lane));
#pragma unroll
            for (int dt = 0; dt < DH / 16; ++dt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NCT / 2; ++ks) {
                    acc = mfma16(as_bf16x8(wa[dt][ks]), ub[ks], acc);
                    acc = mfma16(as_bf16x8(wa[dt][ks]), um[ks], acc);
                    acc = mfma16(as_bf16x8(wa[dt][ks]), ul[ks], acc);
                }
                if (jrow == jj) *reinterpret_cast<floatx4*>(blk + (dt * 64 + lane) * 4) = acc;
            }
        }
    }
    block_sync();   // every unit's partial is written
    // sum the four partials: (row tile, d tile) pairs are dealt round-robin over all waves
    for (int pr_ = wave; pr_ < na * 8; pr_ += NS + NV) {
        const int rt = pr_ >> 3, dt = pr_ & 7;
        floatx4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < NV; ++v)
            sum += *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(bufp(v)) +
                                                     (((rt * 8) + dt) * 64 + lane) * 4);
        const int rho = z * R + 16 * rt + r16;
        const int s = rho / h_q, h = rho - (rho / h_q) * h_q;
        const int d0 = dt * 16 + q4 * 4;
        if (direct) {
            u32x2 o;
            o[0] = pack2f(sum[0], sum[1]);
            o[1] = pack2f(sum[2], sum[3]);
            *reinterpret_cast<u32x2*>(out + (((size_t)b * s_q + s) * h_q + h) * DH + d0) = o;
        } else {
            const size_t prow = ((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h;
            *reinterpret_cast<floatx4*>(part_o + prow * DH + d0) = sum;
        }
    }
}

template <int NS>
hipError_t launch_absorb_t(const DecodeArgs& a, int nz, hipStream_t st) {
    const int pairs = a.n_split * a.batch;
    dim3 grid(((pairs + 7) / 8) * 8 * nz);
    // work items that run at once
    static const int per_cu = blocks_per_cu(absorb_decode_kernel<NS>, (NS + NV) * 64);
    const int cap = per_cu * a.cus / nz;
    hipLaunchKernelGGL((absorb_decode_kernel<NS>), grid, dim3((NS + NV) * 64), 0, st,
                       (const unsigned char*)a.qhat, (const u16*)a.wpack, (const u16*)a.cache, a.bstride,
                       a.ctx_lens, a.max_ctx, a.h_q, a.g, a.s_q, a.chunk, a.n_split, nz, cap, a.batch,
                       a.scale * kLog2e, a.part_o, a.part_lse, (u16*)a.out, a.lse);
    return hipGetLastError();
}

}  // namespace

int absorb_block_rows(int query_rows) { return query_rows < 64 ? query_rows : 64; }

size_t absorb_qrec_bytes() { return QREC; }

size_t absorb_wpack_bytes(int g) { return (size_t)g * DH * RK * sizeof(u16); }

hipError_t launch_absorb_bf16(const DecodeArgs& a, hipStream_t st) {
    const int hpg = a.h_q / a.g;
    const int rows_per_group = a.batch * a.s_q * hpg;
    dim3 pgrid((rows_per_group + 63) / 64, a.g, RK / PRO_COLS);
    hipLaunchKernelGGL(absorb_prologue_kernel, pgrid, dim3(256), 0, st,
                       (const u16*)a.q_nope, (const u16*)a.q_rope, (const u16*)a.w_uk, (const u16*)a.w_uv,
                       (unsigned char*)a.qhat, (u16*)a.wpack, a.batch, a.h_q, a.g, a.s_q, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int RQ = a.s_q * a.h_q;
    const int rows = absorb_block_rows(RQ);
    const int nz = (RQ + rows - 1) / rows;
    e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    switch (rows / 16) {
        case 1: e = launch_absorb_t<1>(a, nz, st); break;
        case 2: e = launch_absorb_t<2>(a, nz, st); break;
        case 3: e = launch_absorb_t<3>(a, nz, st); break;
        default: e = launch_absorb_t<4>(a, nz, st); break;
    }
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

}  // namespace gqla
