// backward_gfx950.hip -- gradients of the GDLA attention core of a full
// prefill with respect to its six inputs (q_signal, q_noise, k, v, lambda,
// gate).
//
// The forward (aitrends.kr, GDLA paragraphs) per KV head j: signal heads
// 4j..4j+3 and noise head j attend with K_j, V_j; D = H_S - lambda (.)
// Repeat_4(H_N); out = gate (.) D.  With dO the gradient of the output:
//   dgate = dO (.) D,  dD = gate (.) dO,
//   dlambda_h = -sum_d dD_h H_N,j,   dH_S,h = dD_h,   dH_N,j = -sum_h lambda_h dD_h,
// and for every head, with P its softmax weights and delta = rowsum(dH (.) H),
//   dV_j += P^T dH,   dS = P (.) (dH V_j^T - delta),   dQ = scale dS K_j,
//   dK_j += scale dS^T Q.
// The forward is recomputed first (the pages' long-context training recomputes
// activations operator by operator): the prefill kernel in its saving mode
// writes H_S, H_N and each row's log2-sum-exp, so that P = exp2(scale log2(e)
// S - lse) is rebuilt exactly in the passes below.
//
// Kernels (all deterministic: every output element is summed by one lane):
//   bwd_pre_kernel   the element-wise differential/gate part, dH and delta;
//   bwd_dkdv_kernel  per (sequence, KV head, 128-key block): wave w of 4 owns
//                    32 keys and walks every query tile that sees them for all
//                    5 heads;
//   bwd_dq_kernel    per (sequence, KV head, 128-query tile): wave w of 8 owns
//                    16 queries and walks every key block they see, head by
//                    head.
// dK/dV: one wave per SIMD with 512 registers, which hold the K and V
// fragments and the dK and dV sums of 32 keys, so each fragment read from LDS
// serves two products.  dQ: two waves per SIMD (at most 256 registers each):
// while one wave waits on an LDS read or its exponentials, the other's
// products keep the matrix core busy.
// Products are bf16 MFMA (16x16x32) with fp32 accumulation; operands that
// have to be transposed come from LDS through the transposing reads.
#include "gdla_device.h"
#include "gdla_launch.h"

namespace gdla {

constexpr int BW_T = 64;                   // query tile and key block
constexpr int BW_THREADS = 256;            // element-wise kernel
constexpr int BW_GW = 8;                   // waves of a dQ workgroup (two per SIMD)
constexpr int BW_GRAD_THREADS = 64 * BW_GW;
constexpr int BW_OWN = 16 * BW_GW;         // keys (dK/dV) or queries (dQ) of a gradient workgroup
// LDS rows padded by 32 bytes: the 16 rows a fragment read or a transposing
// read touches then fall in distinct banks (a 16-byte pad leaves ~40 % of the
// LDS cycles in bank conflicts)
constexpr int BW_QROW = D_QK + 16;         // LDS row of a Q or K tile (bf16)
constexpr int BW_VROW = D_V + 16;          // LDS row of a dH or V tile (bf16)

struct BwdParams {
    const __bf16 *qs, *qn, *k, *v, *lam, *gate, *dout;
    const __bf16 *hs, *hn;                 // saved per-head outputs
    const float *lse;                      // saved log2-sum-exp, [rows][n_sig + n_kv]
    __bf16 *dhs, *dhn;                     // dH of the signal and noise heads
    float *delta;                          // rowsum(dH (.) H), [rows][n_sig + n_kv]
    __bf16 *dqs, *dqn, *dk, *dv, *dlam, *dgate;
    int B, T, n_kv, window;
    float scale, scale_log2;
};

typedef short bw_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bw_s16x4 bw_lds_s16x4_t;

__device__ __forceinline__ bw_s16x4 bw_read_tr16(const __bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_s16x4_t *)(p));
}

// A operand of M^T for a row-major LDS matrix M (row stride rs): 16 columns
// col0 .. col0+15 by the 32 rows row0 + {4g+e} and row0 + 16 + {4g+e} (the
// k order of a B operand packed from two 16-row C blocks)
__device__ __forceinline__ bf16x8 bw_tr_a(const __bf16 *m, int rs, int row0, int col0, int r, int g) {
    const __bf16 *p = m + (row0 + 4 * g + (r >> 2)) * rs + col0 + 4 * (r & 3);
    const bw_s16x4 v8[2] = {bw_read_tr16(p), bw_read_tr16(p + 16 * rs)};
    return __builtin_bit_cast(bf16x8, v8);
}


// ---- 64-row tiles are copied HBM -> LDS with direct (register-free) 16-byte
// loads into a ring of three slots, two steps ahead of the step that reads
// them.  The copy is written as a statement the compiler does not model as an
// LDS write: otherwise it waits for every copy in flight before the next LDS
// read, which would leave no copy in flight under the products.  The kernels
// order copies and reads themselves (vmcnt waits and a barrier before a slot
// is read, and a slot is refilled only after the barrier that ends its last
// reader).  Lane l of a copy writes lds_addr + size*l; the LDS address goes to
// M0; the nop is the wait state an LDS-DMA load needs after M0 is written.
typedef int bw_i32x4 __attribute__((ext_vector_type(4)));

// raw buffer resource over `bytes` bytes from `base`: reads at byte offsets
// >= bytes return zeros (rows past the sequence end)
__device__ __forceinline__ bw_i32x4 bw_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return bw_i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}
__device__ __forceinline__ void bw_copy16(const bw_i32x4 &rsrc, uint32_t byte_off, uint32_t lds_addr) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(byte_off), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void bw_copy4(const bw_i32x4 &rsrc, uint32_t byte_off, uint32_t lds_addr) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :: "v"(byte_off), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}
template <typename T>
__device__ __forceinline__ uint32_t bw_lds(const T *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T *)p;
}

// One 64-row tile of COLS bf16 per row into LDS rows of RS bf16 (RS - COLS
// pad): each copy instruction covers whole rows (2 rows of 26 chunks for the
// 192-wide tiles, 3 rows of 18 chunks for the 128-wide ones), so a lane's row
// and chunk within an instruction are fixed and the pad chunks are skipped;
// wave w of GW issues instructions w, w+GW, ...
template <int COLS, int RS, int GW>
struct BwTileCopy {
    static constexpr int CH = RS / 8;                 // 16-byte chunks per LDS row
    static constexpr int ROWS = 64 / CH;              // rows per instruction
    static constexpr int N = (BW_T + ROWS - 1) / ROWS;
    static constexpr int PER_WAVE = (N + GW - 1) / GW;
    int lr, ch;
    __device__ __forceinline__ void init(int lane) {
        lr = lane / CH;
        ch = lane % CH;
    }
    // rows of the tile start at `rsrc`, `row_bytes` apart; lds_tile: LDS byte address of the slot
    __device__ __forceinline__ void issue(const bw_i32x4 &rsrc, uint32_t row_bytes, uint32_t lds_tile, int wave) const {
#pragma unroll
        for (int c = 0; c < PER_WAVE; ++c) {
            const int row0 = ROWS * (wave + GW * c);
            if (row0 < BW_T && lr < ROWS && ch < COLS / 8 && row0 + lr < BW_T)
                bw_copy16(rsrc, (uint32_t)(row0 + lr) * row_bytes + 16 * ch, lds_tile + (uint32_t)(row0 * RS * 2));
        }
    }
};
static_assert(64 / (BW_QROW / 8) == 2 && 64 / (BW_VROW / 8) == 3, "rows per copy");

// ---- 1. element-wise part.  32 lanes per (token, KV head j), 4 values each.
__global__ __launch_bounds__(BW_THREADS) void bwd_pre_kernel(BwdParams p) {
    const int lane32 = threadIdx.x & 31;
    const long unit = (long)blockIdx.x * (BW_THREADS / 32) + (threadIdx.x >> 5);
    const long n_units = (long)p.B * p.T * p.n_kv;
    if (unit >= n_units) return;                 // whole 32-lane groups leave together
    const int n_sig = p.n_kv * GROUP, n_h = n_sig + p.n_kv;
    const long tok = unit / p.n_kv;
    const int j = (int)(unit % p.n_kv), d0 = 4 * lane32;
    auto ld4 = [](const __bf16 *q, float f[4]) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(q);
        f[0] = bf16_lo(w[0]); f[1] = bf16_hi(w[0]); f[2] = bf16_lo(w[1]); f[3] = bf16_hi(w[1]);
    };
    float hn[4], dhn[4] = {0.f, 0.f, 0.f, 0.f};
    ld4(p.hn + (tok * p.n_kv + j) * D_V + d0, hn);
    float red[2 * GROUP + 1];                    // dlambda_h, delta_h (signal), delta (noise)
#pragma unroll
    for (int h = 0; h < GROUP; ++h) {
        const long row = (tok * n_sig + GROUP * j + h) * D_V + d0;
        float o[4], gt[4], hs[4];
        ld4(p.dout + row, o);
        ld4(p.gate + row, gt);
        ld4(p.hs + row, hs);
        const float lam = (float)p.lam[tok * n_sig + GROUP * j + h];
        float dd[4], dg[4], dl = 0.f, de = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dd[e] = gt[e] * o[e];
            dg[e] = o[e] * fmaf(-lam, hn[e], hs[e]);
            dl -= dd[e] * hn[e];
            dhn[e] -= lam * dd[e];
        }
        const u32x2 ddw = {pack_bf16x2(dd[0], dd[1]), pack_bf16x2(dd[2], dd[3])};
        *reinterpret_cast<u32x2 *>(p.dhs + row) = ddw;
        *reinterpret_cast<u32x2 *>(p.dgate + row) = u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
        // delta from the dH the products below use (bf16)
        de = bf16_lo(ddw[0]) * hs[0] + bf16_hi(ddw[0]) * hs[1] + bf16_lo(ddw[1]) * hs[2] + bf16_hi(ddw[1]) * hs[3];
        red[h] = dl;
        red[GROUP + h] = de;
    }
    const u32x2 dnw = {pack_bf16x2(dhn[0], dhn[1]), pack_bf16x2(dhn[2], dhn[3])};
    *reinterpret_cast<u32x2 *>(p.dhn + (tok * p.n_kv + j) * D_V + d0) = dnw;
    red[2 * GROUP] = bf16_lo(dnw[0]) * hn[0] + bf16_hi(dnw[0]) * hn[1] + bf16_lo(dnw[1]) * hn[2] +
                     bf16_hi(dnw[1]) * hn[3];
#pragma unroll
    for (int i = 0; i < 2 * GROUP + 1; ++i)
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) red[i] += __shfl_xor(red[i], o);
    if (lane32 == 0) {
#pragma unroll
        for (int h = 0; h < GROUP; ++h) {
            p.dlam[tok * n_sig + GROUP * j + h] = (__bf16)red[h];
            p.delta[tok * n_h + GROUP * j + h] = red[GROUP + h];
        }
        p.delta[tok * n_h + n_sig + j] = red[2 * GROUP];
    }
}

// head h of group j (0..3 signal, 4 noise): its query rows, dH rows and column
// in lse / delta
struct BwHead {
    const __bf16 *q, *dh;
    long q_stride, dh_stride;    // elements between consecutive tokens
    int col;
};
__device__ __forceinline__ BwHead bw_head(const BwdParams &p, int b, int j, int h) {
    const int n_sig = p.n_kv * GROUP;
    BwHead x;
    const long tok0 = (long)b * p.T;
    if (h < GROUP) {
        x.q = p.qs + (tok0 * n_sig + GROUP * j + h) * D_QK;
        x.dh = p.dhs + (tok0 * n_sig + GROUP * j + h) * D_V;
        x.q_stride = (long)n_sig * D_QK;
        x.dh_stride = (long)n_sig * D_V;
        x.col = GROUP * j + h;
    } else {
        x.q = p.qn + (tok0 * p.n_kv + j) * D_QK;
        x.dh = p.dhn + (tok0 * p.n_kv + j) * D_V;
        x.q_stride = (long)p.n_kv * D_QK;
        x.dh_stride = (long)p.n_kv * D_V;
        x.col = n_sig + j;
    }
    return x;
}

// ---- 2. dK, dV.  Workgroup (KV head j, 128-key block, sequence b), 4 waves,
// one per SIMD; wave w owns the 32 keys kb0 + 32w .. +31 as two 16-key blocks
// (the first query tile of the block sees none of the keys of waves 2, 3:
// their weights there are 0), so each fragment of Q, dH, Q^T or dH^T read
// from LDS serves two products.  Steps: (query tile, head) for every query
// tile that sees a key of the block and each of the 5 heads; the Q and dH
// tiles, the log2-sum-exp and delta of a step are copied two steps ahead into
// a ring of three LDS slots.  In C layout lane (r, g) holds element [query
// 16qb + 4g + e][key r] of S, P, dP, dS.
constexpr int BW_DK_GW = 4;                       // waves of a dK/dV workgroup
constexpr int BW_DK_THREADS = 64 * BW_DK_GW;
constexpr int BW_DK_KB = BW_OWN / (16 * BW_DK_GW); // 16-key blocks per wave (2)
__global__ __launch_bounds__(BW_DK_THREADS, 1) void bwd_dkdv_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 Qs[3][BW_T * BW_QROW];
    __shared__ __attribute__((aligned(16))) __bf16 Hs[3][BW_T * BW_VROW];
    __shared__ __attribute__((aligned(16))) float lse_s[3][BW_T], dl_s[3][BW_T];
    // the KV head is the fastest grid index, so the workgroups are dispatched
    // longest first (key block 0 sees every query tile)
    const int j = blockIdx.x, kb0 = blockIdx.y * BW_OWN, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 15, g = lane >> 4;
    const int n_h = p.n_kv * HEADS, T = p.T;
    int key[BW_DK_KB];
    long kvrow[BW_DK_KB];
#pragma unroll
    for (int s = 0; s < BW_DK_KB; ++s) {
        key[s] = kb0 + 16 * (BW_DK_KB * wave + s) + r;
        kvrow[s] = ((long)b * T + (key[s] < T ? key[s] : 0)) * p.n_kv + j;
    }
    // B operands K_w^T (lane: K[key r][32kk + 8g ..]) and V_w^T of both key blocks
    bf16x8 kf[BW_DK_KB][D_QK / 32], vf[BW_DK_KB][D_V / 32];
    {
        const u32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < BW_DK_KB; ++s) {
#pragma unroll
            for (int kk = 0; kk < D_QK / 32; ++kk)
                kf[s][kk] = __builtin_bit_cast(bf16x8, key[s] < T ? ldg16(p.k + kvrow[s] * D_QK + 32 * kk + 8 * g) : z);
#pragma unroll
            for (int kk = 0; kk < D_V / 32; ++kk)
                vf[s][kk] = __builtin_bit_cast(bf16x8, key[s] < T ? ldg16(p.v + kvrow[s] * D_V + 32 * kk + 8 * g) : z);
        }
    }
    f32x4 dv[BW_DK_KB][D_V / 16], dk[BW_DK_KB][D_QK / 16];
#pragma unroll
    for (int s = 0; s < BW_DK_KB; ++s) {
#pragma unroll
        for (int i = 0; i < D_V / 16; ++i) dv[s][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < D_QK / 16; ++i) dk[s][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // query tiles that see a key of this block
    const int qt_lo = kb0 / BW_T;
    int qt_hi = (T - 1) / BW_T;
    if (p.window > 0) qt_hi = min(qt_hi, (kb0 + BW_OWN - 1 + p.window - 1) / BW_T);
    const int n_steps = (qt_hi - qt_lo + 1) * HEADS;
    BwTileCopy<D_QK, BW_QROW, BW_DK_GW> cq;
    BwTileCopy<D_V, BW_VROW, BW_DK_GW> ch;
    cq.init(lane);
    ch.init(lane);
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    // the copies of step it into slot it % 3
    auto issue = [&](int it) {
        const int slot = it % 3, q0 = (qt_lo + it / HEADS) * BW_T, n_valid = min(BW_T, T - q0);
        const BwHead hd = bw_head(p, b, j, it % HEADS);
        const uint32_t qrb = (uint32_t)hd.q_stride * 2, hrb = (uint32_t)hd.dh_stride * 2;
        cq.issue(bw_rsrc(hd.q + (long)q0 * hd.q_stride, (uint32_t)n_valid * qrb), qrb, bw_lds(Qs[slot]), uwave);
        ch.issue(bw_rsrc(hd.dh + (long)q0 * hd.dh_stride, (uint32_t)n_valid * hrb), hrb, bw_lds(Hs[slot]), uwave);
        // the rows' log2-sum-exp (wave 0) and delta (wave 1), one float per lane
        const long row0 = (long)b * T + q0;
        if (uwave < 2)
            bw_copy4(bw_rsrc((uwave == 0 ? p.lse : p.delta) + row0 * n_h + hd.col, (uint32_t)(n_valid * n_h * 4)),
                     (uint32_t)(lane * n_h * 4), uwave == 0 ? bw_lds(lse_s[slot]) : bw_lds(dl_s[slot]));
    };
    issue(0);
    if (n_steps > 1) issue(1);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    for (int it = 0; it < n_steps; ++it) {
        const int buf = it % 3, q0 = (qt_lo + it / HEADS) * BW_T;
        const __bf16 *qs_ = Qs[buf], *hs_ = Hs[buf];
        // Two halves of 32 queries (16-query blocks 2i, 2i+1): S = Q K_w^T and
        // dP = dH V_w^T for both key blocks from one read of each fragment,
        // then P and dS packed as B operands over the pair, then dV^T += dH^T P
        // and dK^T += Q^T dS, each transposed fragment serving both key
        // blocks.  The rows' log2-sum-exp and delta are read first and the
        // weight is computed for every element, then selected (no branch per
        // element).  A pair is visible when 0 <= q - key < window (one unsigned
        // compare); rows past the sequence end need no test: their Q, dH and
        // delta read as zeros, so they add nothing to dV or dK whatever their
        // weight.
        const uint32_t wlim = p.window == 0 ? 0x7fffffffu : (uint32_t)p.window;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t pw[BW_DK_KB][2][2], sw[BW_DK_KB][2][2];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int qb = 2 * i + hb;
                const __bf16 *qa = qs_ + (16 * qb + r) * BW_QROW + 8 * g;
                const __bf16 *ha = hs_ + (16 * qb + r) * BW_VROW + 8 * g;
                f32x4 sv[BW_DK_KB], dpv[BW_DK_KB];
#pragma unroll
                for (int s = 0; s < BW_DK_KB; ++s) sv[s] = dpv[s] = zero4;
#pragma unroll
                for (int kk = 0; kk < D_QK / 32; ++kk) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(qa + 32 * kk);
#pragma unroll
                    for (int s = 0; s < BW_DK_KB; ++s) sv[s] = mfma16(a, kf[s][kk], sv[s]);
                }
#pragma unroll
                for (int kk = 0; kk < D_V / 32; ++kk) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ha + 32 * kk);
#pragma unroll
                    for (int s = 0; s < BW_DK_KB; ++s) dpv[s] = mfma16(a, vf[s][kk], dpv[s]);
                }
                const float4 lse4 = *reinterpret_cast<const float4 *>(&lse_s[buf][16 * qb + 4 * g]);
                const float4 dl4 = *reinterpret_cast<const float4 *>(&dl_s[buf][16 * qb + 4 * g]);
                const float ls[4] = {lse4.x, lse4.y, lse4.z, lse4.w};
                const float dls[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
#pragma unroll
                for (int s = 0; s < BW_DK_KB; ++s) {
                    float pv[4], dsv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = fast_exp2(fmaf(sv[s][e], p.scale_log2, -ls[e]));
                        pv[e] = (uint32_t)(q0 + 16 * qb + 4 * g + e - key[s]) < wlim ? x : 0.f;
                        dsv[e] = pv[e] * (dpv[s][e] - dls[e]);
                    }
                    pw[s][hb][0] = pack_bf16x2(pv[0], pv[1]);
                    pw[s][hb][1] = pack_bf16x2(pv[2], pv[3]);
                    sw[s][hb][0] = pack_bf16x2(dsv[0], dsv[1]);
                    sw[s][hb][1] = pack_bf16x2(dsv[2], dsv[3]);
                }
            }
            bf16x8 pb[BW_DK_KB], sb[BW_DK_KB];
#pragma unroll
            for (int s = 0; s < BW_DK_KB; ++s) {
                pb[s] = __builtin_bit_cast(bf16x8, (u32x4{pw[s][0][0], pw[s][0][1], pw[s][1][0], pw[s][1][1]}));
                sb[s] = __builtin_bit_cast(bf16x8, (u32x4{sw[s][0][0], sw[s][0][1], sw[s][1][0], sw[s][1][1]}));
            }
#pragma unroll
            for (int db = 0; db < D_V / 16; ++db) {
                const bf16x8 a = bw_tr_a(hs_, BW_VROW, 32 * i, 16 * db, r, g);
#pragma unroll
                for (int s = 0; s < BW_DK_KB; ++s) dv[s][db] = mfma16(a, pb[s], dv[s][db]);
            }
#pragma unroll
            for (int db = 0; db < D_QK / 16; ++db) {
                const bf16x8 a = bw_tr_a(qs_, BW_QROW, 32 * i, 16 * db, r, g);
#pragma unroll
                for (int s = 0; s < BW_DK_KB; ++s) dk[s][db] = mfma16(a, sb[s], dk[s][db]);
            }
        }
        // step it+2 into the slot of step it-1, which every wave finished
        // before the previous barrier; then step it+1 must have landed (only
        // the copies just issued -- 13 to 15 per wave -- may stay in flight)
        // before the bare barrier
        if (it + 2 < n_steps) {
            issue(it + 2);
            __builtin_amdgcn_s_waitcnt(0x007D);   // vmcnt(13) lgkmcnt(0)
        } else {
            __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    // lane (r, g) holds dV[key r][16db + 4g + e] and dK[key r][16db + 4g + e] / scale
#pragma unroll
    for (int s = 0; s < BW_DK_KB; ++s) {
        if (key[s] >= T) continue;
#pragma unroll
        for (int db = 0; db < D_V / 16; ++db)
            *reinterpret_cast<u32x2 *>(p.dv + kvrow[s] * D_V + 16 * db + 4 * g) =
                u32x2{pack_bf16x2(dv[s][db][0], dv[s][db][1]), pack_bf16x2(dv[s][db][2], dv[s][db][3])};
#pragma unroll
        for (int db = 0; db < D_QK / 16; ++db)
            *reinterpret_cast<u32x2 *>(p.dk + kvrow[s] * D_QK + 16 * db + 4 * g) =
                u32x2{pack_bf16x2(dk[s][db][0] * p.scale, dk[s][db][1] * p.scale),
                      pack_bf16x2(dk[s][db][2] * p.scale, dk[s][db][3] * p.scale)};
    }
}

// ---- 3. dQ.  Workgroup (KV head j, 128-query tile, sequence b); wave w owns
// queries q0 + 16w .. +15 (the last key block of the tile is hidden from the
// queries of waves 0..3: their weights there are 0).  Steps: (head, key block) over the 5 heads and the
// key blocks the tile sees; the K and V tiles of a step are copied two steps
// ahead into a ring of three LDS slots.  In C layout lane (r, g) holds element
// [key 16kb + 4g + e][query r] of S^T, P^T, dP^T, dS^T.
__global__ __launch_bounds__(BW_GRAD_THREADS, 1) void bwd_dq_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 Ks[3][BW_T * BW_QROW];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[3][BW_T * BW_VROW];
    // longest first: the last query tiles see the most key blocks
    const int j = blockIdx.x, q0 = (gridDim.y - 1 - blockIdx.y) * BW_OWN, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 15, g = lane >> 4;
    const int n_h = p.n_kv * HEADS, T = p.T;
    const int q = q0 + 16 * wave + r;
    const bool q_ok = q < T;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const int kb_lo = p.window > 0 ? max(0, q0 - p.window + 1) / BW_T : 0;
    const int kb_hi = (min(q0 + BW_OWN, T) - 1) / BW_T;
    const int n_kb = kb_hi - kb_lo + 1, n_steps = HEADS * n_kb;
    const __bf16 *kseq = p.k + ((long)b * T * p.n_kv + j) * D_QK;
    const __bf16 *vseq = p.v + ((long)b * T * p.n_kv + j) * D_V;
    const long kv_qs = (long)p.n_kv * D_QK, kv_vs = (long)p.n_kv * D_V;
    BwTileCopy<D_QK, BW_QROW, BW_GW> ck;
    BwTileCopy<D_V, BW_VROW, BW_GW> cv;
    ck.init(lane);
    cv.init(lane);
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    // the copies of step it (key block kb_lo + it % n_kb) into slot it % 3
    auto issue = [&](int it) {
        const int slot = it % 3, k0 = (kb_lo + it % n_kb) * BW_T, n_valid = min(BW_T, T - k0);
        const uint32_t krb = (uint32_t)kv_qs * 2, vrb = (uint32_t)kv_vs * 2;
        ck.issue(bw_rsrc(kseq + (long)k0 * kv_qs, (uint32_t)n_valid * krb), krb, bw_lds(Ks[slot]), uwave);
        cv.issue(bw_rsrc(vseq + (long)k0 * kv_vs, (uint32_t)n_valid * vrb), vrb, bw_lds(Vs[slot]), uwave);
    };
    issue(0);
    if (n_steps > 1) issue(1);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();

    bf16x8 qf[D_QK / 32], hf[D_V / 32];
    float lse = 0.f, dl = 0.f;
    f32x4 dq[D_QK / 16];
    for (int it = 0; it < n_steps; ++it) {
        const int h = it / n_kb, buf = it % 3, k0 = (kb_lo + it % n_kb) * BW_T;
        const BwHead hd = bw_head(p, b, j, h);
        if (it % n_kb == 0) {
            // a new head: its B operands Q_w^T and dH_w^T (lane: row q, values
            // 32kk + 8g ..), requested before the next step's copy
            const u32x4 z = {0, 0, 0, 0};
            const long qi = q_ok ? q : 0;
#pragma unroll
            for (int kk = 0; kk < D_QK / 32; ++kk)
                qf[kk] = __builtin_bit_cast(bf16x8, q_ok ? ldg16(hd.q + qi * hd.q_stride + 32 * kk + 8 * g) : z);
#pragma unroll
            for (int kk = 0; kk < D_V / 32; ++kk)
                hf[kk] = __builtin_bit_cast(bf16x8, q_ok ? ldg16(hd.dh + qi * hd.dh_stride + 32 * kk + 8 * g) : z);
            const long row = (long)b * T + qi;
            lse = q_ok ? p.lse[row * n_h + hd.col] : 0.f;
            dl = q_ok ? p.delta[row * n_h + hd.col] : 0.f;
#pragma unroll
            for (int i = 0; i < D_QK / 16; ++i) dq[i] = zero4;
        }
        const __bf16 *ks_ = Ks[buf], *vs_ = Vs[buf];
        // a pair is visible when 0 <= q - key < window (one unsigned compare);
        // keys past the sequence end read zero K rows and add nothing to dQ
        const uint32_t wlim = p.window == 0 ? 0x7fffffffu : (uint32_t)p.window;
        uint32_t sw[4][2];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const __bf16 *ka = ks_ + (16 * k4 + r) * BW_QROW + 8 * g;
            const __bf16 *va = vs_ + (16 * k4 + r) * BW_VROW + 8 * g;
            f32x4 stv = zero4, dpt = zero4;
#pragma unroll
            for (int kk = 0; kk < D_QK / 32; ++kk)
                stv = mfma16(*reinterpret_cast<const bf16x8 *>(ka + 32 * kk), qf[kk], stv);
#pragma unroll
            for (int kk = 0; kk < D_V / 32; ++kk)
                dpt = mfma16(*reinterpret_cast<const bf16x8 *>(va + 32 * kk), hf[kk], dpt);
            float dsv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = fast_exp2(fmaf(stv[e], p.scale_log2, -lse));
                const float pv = (uint32_t)(q - (k0 + 16 * k4 + 4 * g + e)) < wlim ? x : 0.f;
                dsv[e] = pv * (dpt[e] - dl);
            }
            sw[k4][0] = pack_bf16x2(dsv[0], dsv[1]);
            sw[k4][1] = pack_bf16x2(dsv[2], dsv[3]);
        }
        // dQ^T += K^T dS^T over the key pairs (blocks 2i, 2i+1)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bf16x8 sb = __builtin_bit_cast(bf16x8, (u32x4{sw[2 * i][0], sw[2 * i][1], sw[2 * i + 1][0],
                                                                sw[2 * i + 1][1]}));
#pragma unroll
            for (int db = 0; db < D_QK / 16; ++db) dq[db] = mfma16(bw_tr_a(ks_, BW_QROW, 32 * i, 16 * db, r, g), sb, dq[db]);
        }
        if (it % n_kb == n_kb - 1 && q_ok) {
            // the head's last key block: lane (r, g) holds dQ[query r][16db + 4g + e] / scale
            __bf16 *dst = h < GROUP ? p.dqs + (((long)b * T + q) * (p.n_kv * GROUP) + GROUP * j + h) * D_QK
                                    : p.dqn + (((long)b * T + q) * p.n_kv + j) * D_QK;
#pragma unroll
            for (int db = 0; db < D_QK / 16; ++db)
                *reinterpret_cast<u32x2 *>(dst + 16 * db + 4 * g) =
                    u32x2{pack_bf16x2(dq[db][0] * p.scale, dq[db][1] * p.scale),
                          pack_bf16x2(dq[db][2] * p.scale, dq[db][3] * p.scale)};
        }
        // step it+2 into the slot of step it-1 (finished by every wave before
        // the previous barrier); step it+1 must have landed before the barrier
        // (the 6 or 7 copies just issued may stay in flight)
        if (it + 2 < n_steps) {
            issue(it + 2);
            __builtin_amdgcn_s_waitcnt(0x0076);   // vmcnt(6) lgkmcnt(0)
        } else {
            __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
}

// workspace: saved H_S | H_N | lse | the recomputed output | dH_S | dH_N | delta
struct BwLayout {
    size_t hs, hn, lse, out, dhs, dhn, delta, total;
};
static BwLayout bw_layout(int B, int T, int n_kv) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t rows = (size_t)B * T, n_sig = (size_t)n_kv * GROUP;
    BwLayout l;
    l.hs = 0;
    l.hn = l.hs + up(rows * n_sig * D_V * 2);
    l.lse = l.hn + up(rows * n_kv * D_V * 2);
    l.out = l.lse + up(rows * (n_sig + n_kv) * 4);
    l.dhs = l.out + up(rows * n_sig * D_V * 2);
    l.dhn = l.dhs + up(rows * n_sig * D_V * 2);
    l.delta = l.dhn + up(rows * n_kv * D_V * 2);
    l.total = l.delta + up(rows * (n_sig + n_kv) * 4);
    return l;
}

size_t backward_workspace_bytes(int B, int T, int n_kv) { return bw_layout(B, T, n_kv).total; }

hipError_t launch_backward(const void *qs, const void *qn, const void *k, const void *v, const void *lam,
                           const void *gate, const void *dout, void *dqs, void *dqn, void *dk, void *dv,
                           void *dlam, void *dgate, void *workspace, int B, int T, int n_kv, int window,
                           float scale, hipStream_t stream) {
    const BwLayout lay = bw_layout(B, T, n_kv);
    char *ws = static_cast<char *>(workspace);
    // 1. the forward again, saving H_S, H_N and the log2-sum-exp
    hipError_t e = launch_prefill(qs, qn, k, v, lam, gate, ws + lay.out, B, T, 0, n_kv, window, scale, stream,
                                  ws + lay.hs, ws + lay.hn, reinterpret_cast<float *>(ws + lay.lse));
    if (e != hipSuccess) return e;
    BwdParams p;
    p.qs = static_cast<const __bf16 *>(qs);
    p.qn = static_cast<const __bf16 *>(qn);
    p.k = static_cast<const __bf16 *>(k);
    p.v = static_cast<const __bf16 *>(v);
    p.lam = static_cast<const __bf16 *>(lam);
    p.gate = static_cast<const __bf16 *>(gate);
    p.dout = static_cast<const __bf16 *>(dout);
    p.hs = reinterpret_cast<const __bf16 *>(ws + lay.hs);
    p.hn = reinterpret_cast<const __bf16 *>(ws + lay.hn);
    p.lse = reinterpret_cast<const float *>(ws + lay.lse);
    p.dhs = reinterpret_cast<__bf16 *>(ws + lay.dhs);
    p.dhn = reinterpret_cast<__bf16 *>(ws + lay.dhn);
    p.delta = reinterpret_cast<float *>(ws + lay.delta);
    p.dqs = static_cast<__bf16 *>(dqs);
    p.dqn = static_cast<__bf16 *>(dqn);
    p.dk = static_cast<__bf16 *>(dk);
    p.dv = static_cast<__bf16 *>(dv);
    p.dlam = static_cast<__bf16 *>(dlam);
    p.dgate = static_cast<__bf16 *>(dgate);
    p.B = B;
    p.T = T;
    p.n_kv = n_kv;
    p.window = window >= T ? 0 : window;
    p.scale = scale;
    p.scale_log2 = scale * LOG2E;
    const long units = (long)B * T * n_kv;
    hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((units + 7) / 8)), dim3(BW_THREADS), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned n_t = (unsigned)((T + BW_OWN - 1) / BW_OWN);
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(n_kv, n_t, B), dim3(BW_DK_THREADS), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(n_kv, n_t, B), dim3(BW_GRAD_THREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdla
