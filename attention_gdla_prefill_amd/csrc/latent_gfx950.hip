// latent_gfx950.hip -- GDLA decode over the latent (compressed) KV cache.
//
// The KV path stores, per token, the normalised compressed KV c (512 values)
// and the decoupled rotary key k^R (64 values), shared by all KV heads; KV head
// j's key and value are the up-projections K_j = [W_uk[j] c ; k^R] and
// V_j = W_uv[j] c (aitrends.kr, GDLA paragraph and head-dimension paragraph:
// compressed KV rank 512, rotary component 64, one expansion to 16 KV heads,
// the rotary key shared by every KV head).  A cache row is 1,152 bytes against
// 10,240 for the expanded K and V of 16 heads.
//
// The up-projections are folded into the query and the output:
//   q.K_j[s] = (W_uk[j]^T q^C) . c_s + q^R . k^R_s
//   sum_s p_s V_j[s] = W_uv[j] (sum_s p_s c_s)
// so every query head attends directly over the 576-value latent rows:
//   1. latent_absorb_kernel: q~ = [W_uk[j]^T q^C ; q^R] for the 80 query heads;
//   2. latent_split_kernel<false>: split-KV attention of all query heads of a
//      sequence over a chunk of its latent rows -- each row read from HBM once
//      for all heads: per chunk the softmax reference m, the sum l and the
//      latent output o~ = sum_s p_s c_s (512 values) per head, with a fixed
//      reference per chunk and a range check; latent_split_kernel<true> redoes
//      the (rare) chunks that failed it against their exact row maxima;
//   3. latent_combine_kernel: log-sum-exp merge of the chunks, the differential
//      combine in the latent space, d~ = o~_S / l_S - lambda * o~_N / l_N (the
//      up-projection is linear, so this equals the combine of the expanded
//      outputs), D = W_uv[j] d~, out = gate * D.
#include "gdla_device.h"
#include "gdla_launch.h"

#include <algorithm>

namespace gdla {

constexpr int LT_C = 512;                 // compressed KV values per row
constexpr int LT_R = 64;                  // rotary key values per row
constexpr int LT_ROW = LT_C + LT_R;       // 576 values, 1152 bytes per cache row
constexpr int LT_KC = D_QK - LT_R;        // 128: content part of a query
constexpr int LT_HEADS_PER_WG = 80;       // query heads one workgroup serves (5 blocks of 16)
constexpr int LT_WAVES = 4;               // one per SIMD; the fifth head block is shared
constexpr int LT_THREADS = 64 * LT_WAVES;
constexpr int LT_BN = 32;                 // keys per LDS tile
constexpr int LT_SLOTS = 4;               // ring of tiles: products of t-1, scores of t, copies of t+1, t+2
constexpr int LT_AHEAD = 2;               // tiles copied ahead
constexpr int LT_KK = LT_ROW / 32;        // 18 MFMA k-steps over a latent row
constexpr int LT_BLOCKS = LT_HEADS_PER_WG / 16;           // 5 head blocks per workgroup
constexpr int LT_CQ = LT_C / 16 / LT_WAVES;               // 8: latent 16-blocks per wave
constexpr int LT_COPIES = (LT_BN + LT_BN / 8) / LT_WAVES; // 9 copy instructions per wave per tile
constexpr int LT_QB = 6;                  // k-steps whose A fragments are read together
constexpr int LT_QK_AHEAD = 6;            // A-fragment reads kept in flight ahead of their products
static_assert(LT_KK % LT_QB == 0, "k-step batches");
static_assert(LT_BN / 8 == LT_WAVES && LT_COPIES == LT_BN / LT_WAVES + 1, "copies split evenly over the waves");
// LDS rows: the c part with a 32-byte pad (conflict-free 16-row fragment reads),
// the rotary part packed (8 rows per copy instruction)
constexpr int LT_CS = LT_C + 16;          // bf16 per c row in LDS (1056 bytes)
constexpr int LT_CHUNK = 8192;            // target keys per workgroup (split)

struct LatentParams {
    const __bf16 *qs, *qn, *lat, *wuk, *wuv, *lam, *gate;
    const int32_t *cu;
    __bf16 *out;
    __bf16 *qt;              // workspace: absorbed queries [B][n_q][576]
    float *part_ml;          // workspace: [B][n_split][n_q][2]  (m in log2 units, l)
    float *part_o;           // workspace: [B][n_split][n_q][512]
    int32_t *redo;           // workspace: [B][n_split][n_hg] chunk needs the exact-maxima redo
    int32_t *order;          // workspace: [B] sequences by visible length, longest first
    int B, n_kv, n_split, window;
    int sorted;              // the split kernels take sequence order[blockIdx.y] (B <= LT_SORT_MAX)
    float scale_log2;
};

// ---- 1. absorbed queries.  Workgroup (KV head j, sequence b), 256 threads:
// thread t forms q~[2t] and q~[2t+1] of the 5 heads of group j (10 dot
// products of 128), reading columns 2t, 2t+1 of W_uk[j] as
// one 4-byte word per row.
constexpr int LT_ABS_SEQ = 1;
constexpr int LT_ABS_ROWS = LT_ABS_SEQ * HEADS;     // 5 query rows per workgroup
constexpr int LT_ABS_THREADS = LT_C / 2;
constexpr int LT_SORT_MAX = 4096;     // batches up to this size are dispatched longest first

__device__ __forceinline__ int lt_visible(const LatentParams &p, int b) {
    const int L = p.cu[b + 1] - p.cu[b];
    return p.window > 0 ? min(L, p.window) : L;
}

__global__ __launch_bounds__(LT_ABS_THREADS) void latent_absorb_kernel(LatentParams p) {
    __shared__ __attribute__((aligned(16))) float qc[LT_ABS_ROWS][LT_KC];
    __shared__ int n_longer;
    const int j = blockIdx.x, b0 = blockIdx.y * LT_ABS_SEQ, t = threadIdx.x;
    const int n_sig = p.n_kv * GROUP, n_q = n_sig + p.n_kv;
    if (p.sorted && j == 0) {
        // the rank of sequence b0 by visible length, longest first (ties by
        // index): the split kernels work through the long chunks first, so the
        // short ones fill the tail
        if (t == 0) n_longer = 0;
        __syncthreads();
        const int mine = lt_visible(p, b0);
        int c = 0;
        for (int o = t; o < p.B; o += LT_ABS_THREADS) {
            const int v = lt_visible(p, o);
            c += (v > mine || (v == mine && o < b0)) ? 1 : 0;
        }
        atomicAdd(&n_longer, c);
        __syncthreads();
        if (t == 0) p.order[n_longer] = b0;
    }
    auto q_src = [&](int b, int h) {
        return h < GROUP ? p.qs + ((long)b * n_sig + GROUP * j + h) * D_QK : p.qn + ((long)b * p.n_kv + j) * D_QK;
    };
    // content parts of the 5 queries of group j for the 4 sequences
    for (int i = t; i < LT_ABS_ROWS * LT_KC; i += LT_ABS_THREADS) {
        const int row = i / LT_KC, d = i % LT_KC, b = b0 + row / HEADS;
        qc[row][d] = b < p.B ? (float)q_src(b, row % HEADS)[d] : 0.f;
    }
    __syncthreads();
    float acc[LT_ABS_ROWS][2];
#pragma unroll
    for (int i = 0; i < LT_ABS_ROWS; ++i) acc[i][0] = acc[i][1] = 0.f;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(p.wuk + (long)j * LT_KC * LT_C) + t;
    for (int d0 = 0; d0 < LT_KC; d0 += 16) {
        // 16 rows of the column pair in flight per round
        uint32_t wv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) wv[k] = __builtin_nontemporal_load(w + (d0 + k) * (LT_C / 2));
#pragma unroll
        for (int d = 0; d < 16; d += 4)
#pragma unroll
            for (int i = 0; i < LT_ABS_ROWS; ++i) {
                const float4 qv = *reinterpret_cast<const float4 *>(&qc[i][d0 + d]);
                const float q4[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    acc[i][0] = fmaf(q4[k], bf16_lo(wv[d + k]), acc[i][0]);
                    acc[i][1] = fmaf(q4[k], bf16_hi(wv[d + k]), acc[i][1]);
                }
            }
    }
#pragma unroll
    for (int i = 0; i < LT_ABS_ROWS; ++i) {
        const int b = b0 + i / HEADS, h = i % HEADS;
        if (b >= p.B) continue;
        const int q = h < GROUP ? GROUP * j + h : n_sig + j;
        __bf16 *dst = p.qt + ((long)b * n_q + q) * LT_ROW;
        *reinterpret_cast<uint32_t *>(dst + 2 * t) = pack_bf16x2(acc[i][0], acc[i][1]);
        if (t < LT_R / 2)            // the rotary part is copied unchanged
            *reinterpret_cast<uint32_t *>(dst + LT_C + 2 * t) =
                *reinterpret_cast<const uint32_t *>(q_src(b, h) + LT_KC + 2 * t);
    }
}

typedef short lt_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) lt_s16x4 lt_lds_s16x4_t;
typedef int lt_i32x4 __attribute__((ext_vector_type(4)));

// One 16-byte buffer -> LDS copy per lane (lane l writes lds + 16*l; the LDS
// address goes to M0).  Written as a statement the compiler does not model as
// an LDS write: otherwise it would wait for every copy in flight before each
// later LDS read, and the ring could not stream.  The kernel orders the copies
// against the reads itself (vmcnt waits and a barrier before a tile is read).
// The nop is the wait state an LDS-DMA load needs after M0 is written.
__device__ __forceinline__ void lt_copy16(const lt_i32x4 &rsrc, uint32_t byte_off, uint32_t lds_addr) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(byte_off), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ lt_s16x4 lt_read_tr16(const __bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lt_lds_s16x4_t *)(p));
}

// ---- 2. split-KV attention over latent rows.  Workgroup (split, sequence,
// group of 80 query heads = 5 blocks of 16, the MFMA N dimension), 4 waves, one
// per SIMD, walking the chunk in tiles of 32 keys.
//   scores: wave w forms the scores and weights of block w and of the fifth
//     block (the same instructions on the same data in every wave, so the same
//     values), reading the A fragments once for both;
//   outputs: wave w accumulates latent values 128w .. 128w+127 of all five
//     blocks, so each transposing read of the tile serves five products; the
//     weights of blocks 0..3 pass through LDS.
// The products of tile t run after the barrier of tile t+1 (which also orders
// the weight exchange); the copies run two tiles ahead, so the ring still holds
// tile t then.

// the chunk one workgroup walks and its copy addressing
struct LtChunk {
    lt_i32x4 rsrc;           // buffer over the chunk's rows (rows past the sequence end read as zeros)
    uint32_t c_lds, r_lds;   // LDS byte addresses of the two rings
    uint32_t c_off, r_off;   // this lane's byte offsets within a row / a group of 8 rows
    int wave, lane, r, g;
    int k_begin, k_end, n_tiles;
    float c_log2;
};

typedef __bf16 LtCTile[LT_BN * LT_CS];
typedef __bf16 LtRTile[LT_BN * LT_R];
typedef bf16x8 LtPTile[LT_WAVES][64];        // weights of blocks 0..3, one 16-byte B fragment per lane

// Softmax passes over the chunk.  Pass 0: the reference of each head (log2
// units) is the row maximum of the chunk's first tile, kept fixed: a later
// score above it only scales the weights up, and the sums stay in range unless
// scores exceed it by ~62 (log2 units).  Pass 1: exact row maxima of the chunk
// only.  Pass 2: the weights against those exact maxima.
template <int PASS>
__device__ __forceinline__ void lt_pass(const LtChunk &ck, LtCTile *Cring, LtRTile *Rring, LtPTile *Pbuf,
                                        const bf16x8 (&qf)[LT_KK], const bf16x8 (&qf4)[LT_KK],
                                        float &m_ref, float &m4_ref, float &l_part, float &l4_part,
                                        f32x4 (&o)[LT_BLOCKS][LT_CQ]) {
    const int wave = ck.wave, lane = ck.lane, r = ck.r, g = ck.g, n_tiles = ck.n_tiles;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // one instruction copies one row's c part (64 lanes x 16 bytes) or the
    // rotary parts of 8 rows (lane -> row lane/8, 16-byte chunk lane%8): wave w
    // copies the c parts of rows w, w+4, .., w+28 and the rotary parts of rows
    // 8w .. 8w+7
    auto issue_tile = [&](int t) {
        const int slot = t % LT_SLOTS;
        const uint32_t tb = (uint32_t)t * LT_BN * (LT_ROW * 2);
#pragma unroll
        for (int k = 0; k < LT_BN / LT_WAVES; ++k) {
            const int row = wave + LT_WAVES * k;
            lt_copy16(ck.rsrc, tb + row * (LT_ROW * 2) + ck.c_off,
                      ck.c_lds + (uint32_t)(slot * LT_BN * LT_CS + row * LT_CS) * 2);
        }
        lt_copy16(ck.rsrc, tb + 8 * wave * (LT_ROW * 2) + ck.r_off,
                  ck.r_lds + (uint32_t)(slot * LT_BN * LT_R + 8 * wave * LT_R) * 2);
    };
    // o~^T += C^T P^T for tile t over this wave's latent quarter: A = 16 latent
    // values x 32 keys from two transposing reads (lane (r, g) receives
    // C[4g + e][16cb + r] and C[16 + 4g + e][16cb + r]), B = the weights of a block
    auto products = [&](int t, const bf16x8 &pb4) {
        const __bf16 *vrd = Cring[t % LT_SLOTS] + (4 * g + (r >> 2)) * LT_CS + 4 * (r & 3) + 16 * LT_CQ * wave;
        bf16x8 a[LT_CQ];
#pragma unroll
        for (int i = 0; i < LT_CQ; ++i) {
            const lt_s16x4 v8[2] = {lt_read_tr16(vrd + 16 * i), lt_read_tr16(vrd + 16 * LT_CS + 16 * i)};
            a[i] = __builtin_bit_cast(bf16x8, v8);
        }
        bf16x8 pb[LT_BLOCKS];
#pragma unroll
        for (int bk = 0; bk < LT_WAVES; ++bk) pb[bk] = Pbuf[t & 1][bk][lane];
        pb[LT_WAVES] = pb4;
#pragma unroll
        for (int bk = 0; bk < LT_BLOCKS; ++bk)
#pragma unroll
            for (int i = 0; i < LT_CQ; ++i) o[bk][i] = mfma16(a[i], pb[bk], o[bk][i]);
    };

    int next_copy = 0;
    while (next_copy < min(n_tiles, LT_AHEAD)) issue_tile(next_copy++);
    bf16x8 pb4_prev;
    for (int t = 0; t < n_tiles; ++t) {
        // tile t landed for every wave (each wave issues LT_COPIES = 9 copies per
        // tile: vmcnt(9) leaves the one newer tile in flight); every wave is done
        // with iteration t-1: its weights are in LDS, and the products of tile
        // t-2, the last reader of the slot the copy of tile t+2 reuses, are done.
        // A bare barrier: a workgroup fence would also drain the newer copies.
        if (next_copy - 1 - t >= 1) __builtin_amdgcn_s_waitcnt(0x0079);   // vmcnt(9) lgkmcnt(0)
        else __builtin_amdgcn_s_waitcnt(0x0070);                          // vmcnt(0) lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (next_copy < n_tiles) issue_tile(next_copy++);

        const __bf16 *cs = Cring[t % LT_SLOTS], *rs = Rring[t % LT_SLOTS];
        const int kb0 = ck.k_begin + t * LT_BN;
        // S^T = C q~^T for the tile's 32 keys and both head blocks; one A
        // fragment (16 latent rows x 32 values) serves both.  Fragments are read
        // LT_QB k-steps at a time, ahead of their products.
        f32x4 s[2], s4[2];
#pragma unroll
        for (int bt = 0; bt < LT_KK / LT_QB; ++bt) {
            bf16x8 af[LT_QB][2];
#pragma unroll
            for (int j = 0; j < LT_QB; ++j) {
                const int kk = bt * LT_QB + j;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const __bf16 *crow = cs + (16 * kb + r) * LT_CS + 8 * g;
                    const __bf16 *rrow = rs + (16 * kb + r) * LT_R + 8 * g;
                    af[j][kb] = kk < LT_C / 32 ? *reinterpret_cast<const bf16x8 *>(crow + 32 * kk)
                                               : *reinterpret_cast<const bf16x8 *>(rrow + 32 * (kk - LT_C / 32));
                }
            }
#pragma unroll
            for (int j = 0; j < LT_QB; ++j) {
                const int kk = bt * LT_QB + j;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    s[kb] = mfma16(af[j][kb], qf[kk], kk == 0 ? zero4 : s[kb]);
                    s4[kb] = mfma16(af[j][kb], qf4[kk], kk == 0 ? zero4 : s4[kb]);
                }
            }
        }
        // the interleave of the block above: LT_QK_AHEAD fragment reads (LDS)
        // ahead, then two products (MFMA) per read
        __builtin_amdgcn_sched_group_barrier(0x100, LT_QK_AHEAD, 0);
#pragma unroll
        for (int i = 0; i < 2 * LT_KK - LT_QK_AHEAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * LT_QK_AHEAD, 0);
        if (PASS != 1 && t > 0) products(t - 1, pb4_prev);
        // keys past the chunk end are masked; row maxima in log2 units
        float mx = -INFINITY, mx4 = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (kb0 + 16 * kb + 4 * g + e >= ck.k_end) {
                    s[kb][e] = -INFINITY;
                    s4[kb][e] = -INFINITY;
                }
                mx = fmaxf(mx, s[kb][e]);
                mx4 = fmaxf(mx4, s4[kb][e]);
            }
        mx = group4_max(mx) * ck.c_log2;
        mx4 = group4_max(mx4) * ck.c_log2;
        if (PASS == 1) {
            m_ref = fmaxf(m_ref, mx);
            m4_ref = fmaxf(m4_ref, mx4);
            continue;
        }
        if (PASS == 0 && t == 0) {
            m_ref = mx;
            m4_ref = mx4;
        }
        const float mref = m_ref == -INFINITY ? 0.f : m_ref;
        const float mref4 = m4_ref == -INFINITY ? 0.f : m4_ref;
        uint32_t pw[4], pw4[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float pv[4], pv4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[e] = fast_exp2(fmaf(s[kb][e], ck.c_log2, -mref));
                pv4[e] = fast_exp2(fmaf(s4[kb][e], ck.c_log2, -mref4));
            }
            pw[2 * kb] = pack_bf16x2(pv[0], pv[1]);
            pw[2 * kb + 1] = pack_bf16x2(pv[2], pv[3]);
            pw4[2 * kb] = pack_bf16x2(pv4[0], pv4[1]);
            pw4[2 * kb + 1] = pack_bf16x2(pv4[2], pv4[3]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            l_part = sum_bf16x2(pw[i], l_part);
            l4_part = sum_bf16x2(pw4[i], l4_part);
        }
        // this block's weights for the other waves (B fragment: lane (r, g) holds
        // keys 4g..4g+3 and 16+4g..16+4g+3 of head r, the order of the A rows)
        Pbuf[t & 1][wave][lane] = __builtin_bit_cast(bf16x8, (u32x4{pw[0], pw[1], pw[2], pw[3]}));
        pb4_prev = __builtin_bit_cast(bf16x8, (u32x4{pw4[0], pw4[1], pw4[2], pw4[3]}));
    }
    if (PASS != 1 && n_tiles > 0) {
        // the last tile's products, once every wave's weights are in LDS (no
        // copy is in flight: the last tile waited for all)
        __syncthreads();
        products(n_tiles - 1, pb4_prev);
    }
}

// REDO = false: pass 0 over every chunk, then a workgroup-wide range check whose
// outcome goes to p.redo.  REDO = true (launched after it): a workgroup whose
// chunk failed the check runs passes 1 and 2 and rewrites the partials; the
// others exit at once.
template <bool REDO>
__global__ __launch_bounds__(LT_THREADS, 1) void latent_split_kernel(LatentParams p) {
    __shared__ __attribute__((aligned(16))) LtCTile Cring[LT_SLOTS];
    __shared__ __attribute__((aligned(16))) LtRTile Rring[LT_SLOTS];
    __shared__ __attribute__((aligned(16))) LtPTile Pbuf[2];
    __shared__ int range_bad[LT_WAVES];

    const int sp = blockIdx.x, hg = blockIdx.z;
    const int b = p.sorted ? p.order[blockIdx.y] : blockIdx.y;
    int32_t *redo_flag = p.redo + ((long)b * p.n_split + sp) * gridDim.z + hg;
    if (REDO && *(volatile int32_t *)redo_flag == 0) return;
    const int n_sig = p.n_kv * GROUP, n_q = n_sig + p.n_kv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int q0 = hg * LT_HEADS_PER_WG;                                   // first head of block 0
    const int q_row = q0 + 16 * wave + r, q4_row = q0 + 16 * LT_WAVES + r;
    const bool q_ok = q_row < n_q, q4_ok = q4_row < n_q;

    LtChunk ck;
    const int start = p.cu[b];
    const int L = p.cu[b + 1] - start;
    const int vis_lo = p.window > 0 ? max(0, L - p.window) : 0;
    const int n_vis = max(0, L - vis_lo);
    const int chunk = (n_vis + p.n_split - 1) / p.n_split;
    ck.k_begin = vis_lo + sp * chunk;                              // relative to the sequence start
    ck.k_end = min(L, ck.k_begin + chunk);
    ck.n_tiles = ck.k_end > ck.k_begin ? (ck.k_end - ck.k_begin + LT_BN - 1) / LT_BN : 0;
    ck.wave = wave;
    ck.lane = lane;
    ck.r = r;
    ck.g = g;
    ck.c_log2 = p.scale_log2;

    // absorbed queries of this lane's two heads: B operands, lane holds q~[32kk + 8g .. +7]
    bf16x8 qf[LT_KK], qf4[LT_KK];
    {
        const __bf16 *src = p.qt + ((long)b * n_q + (q_ok ? q_row : 0)) * LT_ROW + 8 * g;
        const __bf16 *src4 = p.qt + ((long)b * n_q + (q4_ok ? q4_row : 0)) * LT_ROW + 8 * g;
#pragma unroll
        for (int kk = 0; kk < LT_KK; ++kk) {
            u32x4 w = q_ok ? ldg16(src + 32 * kk) : u32x4{0, 0, 0, 0};
            u32x4 w4 = q4_ok ? ldg16(src4 + 32 * kk) : u32x4{0, 0, 0, 0};
            qf[kk] = __builtin_bit_cast(bf16x8, w);
            qf4[kk] = __builtin_bit_cast(bf16x8, w4);
        }
    }

    const __bf16 *row0 = p.lat + ((long)start + ck.k_begin) * LT_ROW;
    const uint32_t bytes = (uint32_t)max(0, L - ck.k_begin) * (LT_ROW * 2);
    const uint64_t row0a = reinterpret_cast<uint64_t>(row0);
    ck.rsrc = lt_i32x4{(int)(uint32_t)row0a, (int)(uint32_t)(row0a >> 32), (int)bytes, 0x00020000};
    ck.c_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16 *)&Cring[0][0];
    ck.r_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16 *)&Rring[0][0];
    ck.c_off = 16 * lane;
    ck.r_off = (lane / 8) * (LT_ROW * 2) + LT_C * 2 + 16 * (lane % 8);

    // the query fragments are complete before the loop (so the tile loop carries
    // no wait for them, which would also drain the copies in flight)
#pragma unroll
    for (int kk = 0; kk < LT_KK; ++kk) asm volatile("" ::"v"(qf[kk]), "v"(qf4[kk]));

    float m_ref = -INFINITY, m4_ref = -INFINITY, l_part = 0.f, l4_part = 0.f;
    f32x4 o[LT_BLOCKS][LT_CQ];
#pragma unroll
    for (int bk = 0; bk < LT_BLOCKS; ++bk)
#pragma unroll
        for (int i = 0; i < LT_CQ; ++i) o[bk][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!REDO) {
        lt_pass<0>(ck, Cring, Rring, Pbuf, qf, qf4, m_ref, m4_ref, l_part, l4_part, o);
        // range check over the workgroup
        const bool bad = __any(!(l_part <= RESTART_PART_SUM) || !(l4_part <= RESTART_PART_SUM));
        if (lane == 0) range_bad[wave] = bad;
        __syncthreads();
        const int any_bad = range_bad[0] | range_bad[1] | range_bad[2] | range_bad[3];
        if (tid == 0) *redo_flag = any_bad;
        if (any_bad) return;
    } else {
        lt_pass<1>(ck, Cring, Rring, Pbuf, qf, qf4, m_ref, m4_ref, l_part, l4_part, o);
        __syncthreads();          // every wave is done with the ring before it is refilled
        lt_pass<2>(ck, Cring, Rring, Pbuf, qf, qf4, m_ref, m4_ref, l_part, l4_part, o);
    }

    // partials of this chunk: m (log2 units) and l of blocks w and 4, o~ of every
    // block over this wave's latent quarter
    const float l_tot = group4_sum(l_part), l4_tot = group4_sum(l4_part);
    const long pq0 = ((long)b * p.n_split + sp) * n_q + q0;
    if (g == 0 && q_ok) {
        p.part_ml[2 * (pq0 + 16 * wave + r)] = ck.n_tiles > 0 ? m_ref : -INFINITY;
        p.part_ml[2 * (pq0 + 16 * wave + r) + 1] = l_tot;
    }
    if (g == 0 && wave == 0 && q4_ok) {
        p.part_ml[2 * (pq0 + 16 * LT_WAVES + r)] = ck.n_tiles > 0 ? m4_ref : -INFINITY;
        p.part_ml[2 * (pq0 + 16 * LT_WAVES + r) + 1] = l4_tot;
    }
#pragma unroll
    for (int bk = 0; bk < LT_BLOCKS; ++bk) {
        if (q0 + 16 * bk + r >= n_q) continue;
        float *po = p.part_o + (pq0 + 16 * bk + r) * LT_C + 16 * LT_CQ * wave + 4 * g;
#pragma unroll
        for (int i = 0; i < LT_CQ; ++i) *reinterpret_cast<f32x4 *>(po + 16 * i) = o[bk][i];
    }
}

// ---- 3. merge, combine in the latent space, up-project, gate.  Workgroup
// (KV head j, sequence b), 512 threads.
constexpr int LT_MERGE_MAX = 256;          // splits whose weights are staged in LDS at once

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ __launch_bounds__(LT_C) void latent_combine_kernel(LatentParams p) {
    __shared__ float dl[GROUP][LT_C];          // d~ of the 4 signal heads
    __shared__ float wgt[HEADS][LT_MERGE_MAX]; // merge weights of a batch of splits
    __shared__ float head_m[HEADS], head_il[HEADS];
    __shared__ float red[LT_C / D_V][GROUP][D_V];
    const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n_sig = p.n_kv * GROUP, n_q = n_sig + p.n_kv;
    auto head_q = [&](int h) { return h < GROUP ? GROUP * j + h : n_sig + j; };
    // the splits of sequence b that hold keys (the split kernel's chunking)
    const int L = p.cu[b + 1] - p.cu[b];
    const int n_vis = p.window > 0 ? min(L, p.window) : L;
    const int chunk = (n_vis + p.n_split - 1) / p.n_split;
    const int n_valid = chunk > 0 ? (n_vis + chunk - 1) / chunk : 0;
    const long pq_b = (long)b * p.n_split * n_q;
    // 1. per head (wave h): merged maximum and sum over the splits
    if (wv < HEADS) {
        const long q = head_q(wv);
        float m = -INFINITY;
        for (int s = lane; s < n_valid; s += 64) m = fmaxf(m, p.part_ml[2 * (pq_b + (long)s * n_q + q)]);
        m = wave_max(m);
        float l = 0.f;
        for (int s = lane; s < n_valid; s += 64) {
            const float ms = p.part_ml[2 * (pq_b + (long)s * n_q + q)];
            if (ms != -INFINITY) l += fast_exp2(ms - m) * p.part_ml[2 * (pq_b + (long)s * n_q + q) + 1];
        }
        l = wave_sum(l);
        if (lane == 0) {
            head_m[wv] = m;
            head_il[wv] = l > 0.f ? 1.f / l : 0.f;
        }
    }
    __syncthreads();
    // 2. the weighted sum of the chunk outputs, thread c = latent value c
    float acc[HEADS] = {0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_valid; s0 += LT_MERGE_MAX) {
        const int ns = min(LT_MERGE_MAX, n_valid - s0);
        for (int i = tid; i < HEADS * ns; i += LT_C) {
            const int h = i / ns, s = s0 + i % ns;
            const float ms = p.part_ml[2 * (pq_b + (long)s * n_q + head_q(h))];
            wgt[h][i % ns] = ms == -INFINITY ? 0.f : fast_exp2(ms - head_m[h]) * head_il[h];
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < HEADS; ++h) {
            const float *po = p.part_o + (pq_b + (long)s0 * n_q + head_q(h)) * LT_C + tid;
            float a = 0.f;
#pragma unroll 4
            for (int s = 0; s < ns; ++s) a = fmaf(wgt[h][s], po[(long)s * n_q * LT_C], a);
            acc[h] += a;
        }
        __syncthreads();
    }
    {
        const long hrow = (long)b * n_sig + GROUP * j;
#pragma unroll
        for (int h = 0; h < GROUP; ++h) dl[h][tid] = fmaf(-(float)p.lam[hrow + h], acc[GROUP], acc[h]);
    }
    __syncthreads();
    // 3. D[h][d] = sum_c W_uv[j][d][c] d~[h][c]: thread (quarter q4, row d) sums the
    // latent values 128 q4 .. 128 q4 + 127 for the 4 heads (each row of W_uv[j]
    // read once); the quarters then add up through LDS
    {
        const int q4 = tid / D_V, d = tid % D_V, c0 = q4 * (LT_C / 4);
        const __bf16 *w = p.wuv + ((long)j * D_V + d) * LT_C + c0;
        float acc4[GROUP] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int c = 0; c < LT_C / 4; c += 8) {
            const u32x4 wv8 = ldg16(w + c);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int h = 0; h < GROUP; ++h) {
                    acc4[h] = fmaf(bf16_lo(wv8[i]), dl[h][c0 + c + 2 * i], acc4[h]);
                    acc4[h] = fmaf(bf16_hi(wv8[i]), dl[h][c0 + c + 2 * i + 1], acc4[h]);
                }
        }
#pragma unroll
        for (int h = 0; h < GROUP; ++h) red[q4][h][d] = acc4[h];
    }
    __syncthreads();
    const int h = tid / D_V, d = tid % D_V;
    const float D = red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d];
    const long orow = (long)b * n_sig + GROUP * j + h;
    p.out[orow * D_V + d] = (__bf16)((float)p.gate[orow * D_V + d] * D);
}

// ---- window decode over the latent cache (1 <= W <= 128): the whole job of
// one (KV head j, sequence b) in one workgroup, one launch -----------------
//
// With at most 128 visible rows a (sequence, KV head) is a short chain of
// small steps, so the four launches of the split path (each of them at least
// one HBM latency) become four phases of one workgroup, each of which issues
// all of its loads before it waits for any (one memory round trip per phase):
//   1. q~ = [W_uk[j]^T q^C ; q^R] of the 5 heads: thread t takes columns
//      8(t%64) .. +7 of W_uk[j] over rows 32(t/64) .. +31 (a wave reads whole
//      1 KB rows), the four row quarters add up through LDS; rounded to bf16
//      into LDS as the B operand of the scores;
//   2. S^T = L q~^T on the matrix cores, wave w taking rows 32w .. 32w+31 of
//      the window straight from HBM as A fragments; the exact row maxima and
//      sums meet in LDS (no fixed reference, nothing to redo), the weights go
//      to LDS in fp32;
//   3. o~[h][c] = sum_s p_s c_s[c] on the VALU: thread t takes columns
//      8(t%64) .. +7 over rows 32(t/64) .. +31 of the window, the quarters
//      add up through LDS; then the differential combine in the latent
//      space, d~ = o~_S / l_S - lambda o~_N / l_N;
//   4. D = W_uv[j] d~ on the matrix cores (d~ as its bf16 high and low
//      parts, the rows of W_uv[j] as B fragments straight from memory), out =
//      gate * D.
// The row sums are taken over the fp32 weights that enter o~.
constexpr int LW_KEYS = 128;
constexpr int LW_THREADS = 256;
constexpr int LW_QROW = LT_ROW + 8;           // bf16 per absorbed-query row in LDS (16-byte pad)
static_assert(LW_THREADS * 2 == LT_C && LW_THREADS / 64 * 32 == LT_KC && LW_THREADS / 64 * 32 == LW_KEYS,
              "thread / column / row split");

__global__ __launch_bounds__(LW_THREADS, 2) void latent_window_kernel(LatentParams p) {
    __shared__ float qc[HEADS][LT_KC];                                   // content parts of the queries
    __shared__ __attribute__((aligned(16))) __bf16 qt_s[HEADS][LW_QROW]; // absorbed queries
    __shared__ float red_m[4][16], red_l[4][16];
    __shared__ __attribute__((aligned(16))) float pw_s[HEADS][LW_KEYS];  // weights
    __shared__ __attribute__((aligned(16))) float part[4][HEADS][LT_C];  // per-quarter partial sums
    // d~ of the signal heads as bf16 high and low parts (their sum keeps ~16 bits)
    __shared__ __attribute__((aligned(16))) __bf16 dlh[GROUP][LT_C], dll[GROUP][LT_C];

    const int j = blockIdx.x, b = blockIdx.y;
    const int n_kv = p.n_kv, n_sig = n_kv * GROUP;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);

    // ---- loads that need no offsets: cu[b], cu[b+1], W_uk[j], the queries,
    // lambda and the gate
    const auto cu_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(p.cu), 0, (int)((gridDim.y + 1) * 4u),
                                                         0x00020000);
    const u32x2 cuv = __builtin_amdgcn_raw_buffer_load_b64(cu_rs, 4u * b, 0, 0);
    u32x4 wk[32];
    {
        const __bf16 *w = p.wuk + ((long)j * LT_KC + 32 * uwave) * LT_C + 8 * lane;
#pragma unroll
        for (int i = 0; i < 32; ++i) wk[i] = ldg16(w + i * LT_C);
    }
    auto q_src = [&](int h) {
        return h < GROUP ? p.qs + ((long)b * n_sig + GROUP * j + h) * D_QK : p.qn + ((long)b * n_kv + j) * D_QK;
    };
    for (int i = tid; i < HEADS * D_QK; i += LW_THREADS) {
        const int h = i / D_QK, d = i % D_QK;
        const __bf16 v = q_src(h)[d];
        if (d < LT_KC) qc[h][d] = (float)v;
        else qt_s[h][LT_C + d - LT_KC] = v;            // the rotary part is used as it is
    }
    const long orow0 = (long)b * n_sig + GROUP * j;     // signal head 4j
    const u32x2 lw = *reinterpret_cast<const u32x2 *>(p.lam + orow0);     // lambda of the 4 signal heads

    const int start = __builtin_amdgcn_readfirstlane((int)cuv[0]);
    const int L = __builtin_amdgcn_readfirstlane((int)cuv[1]) - start;
    const int n_vis = max(0, min(L, p.window));         // <= LW_KEYS
    const long row0 = (long)start + (L - n_vis);        // first visible cache row
    const auto lat_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16 *>(p.lat + row0 * LT_ROW), 0,
                                                          (int)((uint32_t)n_vis * LT_ROW * 2), 0x00020000);
    __syncthreads();

    // ---- 1. absorbed queries
    {
        float acc[HEADS][8];
#pragma unroll
        for (int h = 0; h < HEADS; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
#pragma unroll
            for (int h = 0; h < HEADS; ++h) {
                const float q = qc[h][32 * uwave + i];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[h][2 * e] = fmaf(q, bf16_lo(wk[i][e]), acc[h][2 * e]);
                    acc[h][2 * e + 1] = fmaf(q, bf16_hi(wk[i][e]), acc[h][2 * e + 1]);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < HEADS; ++h) {
            *reinterpret_cast<f32x4 *>(&part[wave][h][8 * lane]) = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
            *reinterpret_cast<f32x4 *>(&part[wave][h][8 * lane + 4]) = f32x4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < HEADS; ++h) {
        float v[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            v[i] = part[0][h][2 * tid + i] + part[1][h][2 * tid + i] + part[2][h][2 * tid + i] + part[3][h][2 * tid + i];
        *reinterpret_cast<uint32_t *>(&qt_s[h][2 * tid]) = pack_bf16x2(v[0], v[1]);
    }
    __syncthreads();

    // ---- 2. scores of rows 32w + 16kb + r: S^T = L q~^T (columns r >= 5 unused)
    const float c_log2 = p.scale_log2;
    f32x4 s[2];
    {
        bf16x8 la[2][LT_KK];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int k = 0; k < LT_KK; ++k)
                la[kb][k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                    lat_rs, (uint32_t)(32 * uwave + 16 * kb + r) * (LT_ROW * 2) + 64 * k + 16 * g, 0, 0));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[kb][e] = 32 * uwave + 16 * kb + 4 * g + e < n_vis ? 0.f : -INFINITY;
        const __bf16 *qrow = qt_s[r < HEADS ? r : 0] + 8 * g;
        const bool q_on = r < HEADS;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < LT_KK; ++k) {
            const u32x4 qw = *reinterpret_cast<const u32x4 *>(qrow + 32 * k);
            const bf16x8 qb = __builtin_bit_cast(bf16x8, q_on ? qw : z);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = mfma16(la[kb][k], qb, s[kb]);
        }
    }
    {
        const float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                               fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        const float wm = group4_max(mx);
        if (g == 0) red_m[wave][r] = wm;
    }
    __syncthreads();
    {
        const float m = fmaxf(fmaxf(red_m[0][r], red_m[1][r]), fmaxf(red_m[2][r], red_m[3][r]));
        const float m_ref = m == -INFINITY ? 0.f : m * c_log2;
        float l_part = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x4 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[e] = fast_exp2(fmaf(s[kb][e], c_log2, -m_ref));
                l_part += pv[e];
            }
            if (r < HEADS) *reinterpret_cast<f32x4 *>(&pw_s[r][32 * uwave + 16 * kb + 4 * g]) = pv;
        }
        const float wl = group4_sum(l_part);
        if (g == 0) red_l[wave][r] = wl;
    }
    __syncthreads();

    // ---- 3. o~[h][c] = sum_s p_s[h] c_s[c]: columns 8 lane .. +7 over the
    // window rows 32w .. 32w+31 (rows past the window read zeros, weight 0)
    {
        u32x4 cv[32];
#pragma unroll
        for (int i = 0; i < 32; ++i)
            cv[i] = __builtin_amdgcn_raw_buffer_load_b128(lat_rs, (uint32_t)(32 * uwave + i) * (LT_ROW * 2) + 16 * lane,
                                                          0, 0);
        float acc[HEADS][8];
#pragma unroll
        for (int h = 0; h < HEADS; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
#pragma unroll
            for (int h = 0; h < HEADS; ++h) {
                const float w = pw_s[h][32 * uwave + i];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[h][2 * e] = fmaf(w, bf16_lo(cv[i][e]), acc[h][2 * e]);
                    acc[h][2 * e + 1] = fmaf(w, bf16_hi(cv[i][e]), acc[h][2 * e + 1]);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < HEADS; ++h) {
            *reinterpret_cast<f32x4 *>(&part[wave][h][8 * lane]) = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
            *reinterpret_cast<f32x4 *>(&part[wave][h][8 * lane + 4]) = f32x4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
        }
    }
    __syncthreads();
    {
        float inv[HEADS];
#pragma unroll
        for (int h = 0; h < HEADS; ++h) {
            const float l = red_l[0][h] + red_l[1][h] + red_l[2][h] + red_l[3][h];
            inv[h] = l > 0.f ? 1.f / l : 0.f;
        }
        float o[HEADS][2];
#pragma unroll
        for (int h = 0; h < HEADS; ++h)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                o[h][i] = (part[0][h][2 * tid + i] + part[1][h][2 * tid + i] + part[2][h][2 * tid + i] +
                           part[3][h][2 * tid + i]) * inv[h];
        const float lam[GROUP] = {bf16_lo(lw[0]), bf16_hi(lw[0]), bf16_lo(lw[1]), bf16_hi(lw[1])};
#pragma unroll
        for (int h = 0; h < GROUP; ++h) {
            const float v0 = fmaf(-lam[h], o[GROUP][0], o[h][0]), v1 = fmaf(-lam[h], o[GROUP][1], o[h][1]);
            const uint32_t hi = pack_bf16x2(v0, v1);
            *reinterpret_cast<uint32_t *>(&dlh[h][2 * tid]) = hi;
            *reinterpret_cast<uint32_t *>(&dll[h][2 * tid]) = pack_bf16x2(v0 - bf16_lo(hi), v1 - bf16_hi(hi));
        }
    }
    __syncthreads();

    // ---- 4. D = d~ W_uv[j]^T on the matrix cores: M = the 4 signal heads
    // (rows 4..15 zero), N = 16 output columns per block (wave w: blocks 2w,
    // 2w+1), K = the 512 latent values; d~ enters as its bf16 high and low parts,
    // the B fragments are rows of W_uv[j] straight from memory (lane (r, g):
    // W_uv[j][16nb + r][32kk + 8g .. +7])
    {
        u32x4 wv[2][LT_C / 32];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int kk = 0; kk < LT_C / 32; ++kk)
                wv[nb][kk] = ldg16(p.wuv + ((long)j * D_V + 16 * (2 * wave + nb) + r) * LT_C + 32 * kk + 8 * g);
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int kk = 0; kk < LT_C / 32; ++kk) {
            const u32x4 ah = r < GROUP ? *reinterpret_cast<const u32x4 *>(&dlh[r < GROUP ? r : 0][32 * kk + 8 * g]) : z;
            const u32x4 al = r < GROUP ? *reinterpret_cast<const u32x4 *>(&dll[r < GROUP ? r : 0][32 * kk + 8 * g]) : z;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const bf16x8 bw = __builtin_bit_cast(bf16x8, wv[nb][kk]);
                acc[nb] = mfma16(__builtin_bit_cast(bf16x8, ah), bw, acc[nb]);
                acc[nb] = mfma16(__builtin_bit_cast(bf16x8, al), bw, acc[nb]);
            }
        }
        // lane (r, g): rows 4g..4g+3 (heads; g == 0 holds the 4 signal heads),
        // column 16 (2w + nb) + r
        if (g == 0) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int e = 0; e < GROUP; ++e) {
                    const long o_idx = (orow0 + e) * D_V + 16 * (2 * wave + nb) + r;
                    p.out[o_idx] = (__bf16)((float)p.gate[o_idx] * acc[nb][e]);
                }
        }
    }
}

int latent_splits(int max_seqlen_k, int window) {
    const long vis = window > 0 ? (long)std::min(max_seqlen_k, window) : (long)max_seqlen_k;
    const long n = (vis + LT_CHUNK - 1) / LT_CHUNK;
    return (int)std::max(1L, std::min(n, 4096L));
}

// workspace: absorbed queries | chunk maxima and sums | redo flags | sequence order | chunk outputs
struct LtLayout {
    size_t qt, ml, redo, order, o, total;
};
static LtLayout latent_layout(int B, int n_kv, int n_split) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t n_q = (size_t)n_kv * HEADS;
    const size_t n_hg = (n_q + LT_HEADS_PER_WG - 1) / LT_HEADS_PER_WG;
    LtLayout l;
    l.qt = 0;
    l.ml = up((size_t)B * n_q * LT_ROW * 2);
    l.redo = l.ml + up((size_t)B * n_split * n_q * 2 * sizeof(float));
    l.order = l.redo + up((size_t)B * n_split * n_hg * sizeof(int32_t));
    l.o = l.order + up((size_t)B * sizeof(int32_t));
    l.total = l.o + (size_t)B * n_split * n_q * LT_C * sizeof(float);
    return l;
}

size_t latent_workspace_bytes(int B, int n_kv, int n_split) { return latent_layout(B, n_kv, n_split).total; }

hipError_t launch_decode_latent(const void *qs, const void *qn, const void *lat, const int32_t *cu,
                                const void *wuk, const void *wuv, const void *lam, const void *gate,
                                void *out, void *workspace, int B, int n_kv, int n_split, int window,
                                float scale, hipStream_t stream) {
    LatentParams p;
    p.qs = static_cast<const __bf16 *>(qs);
    p.qn = static_cast<const __bf16 *>(qn);
    p.lat = static_cast<const __bf16 *>(lat);
    p.wuk = static_cast<const __bf16 *>(wuk);
    p.wuv = static_cast<const __bf16 *>(wuv);
    p.lam = static_cast<const __bf16 *>(lam);
    p.gate = static_cast<const __bf16 *>(gate);
    p.cu = cu;
    p.out = static_cast<__bf16 *>(out);
    const size_t n_q = (size_t)n_kv * HEADS;
    char *ws = static_cast<char *>(workspace);
    const LtLayout lay = latent_layout(B, n_kv, n_split);
    p.qt = reinterpret_cast<__bf16 *>(ws + lay.qt);
    p.part_ml = reinterpret_cast<float *>(ws + lay.ml);
    p.redo = reinterpret_cast<int32_t *>(ws + lay.redo);
    p.order = reinterpret_cast<int32_t *>(ws + lay.order);
    p.sorted = B <= LT_SORT_MAX;
    p.part_o = reinterpret_cast<float *>(ws + lay.o);
    p.B = B;
    p.n_kv = n_kv;
    p.n_split = n_split;
    p.window = window;
    p.scale_log2 = scale * LOG2E;
    if (window >= 1 && window <= LW_KEYS) {
        // a short window: one workgroup per (KV head, sequence) does it all
        hipLaunchKernelGGL(latent_window_kernel, dim3(n_kv, B), dim3(LW_THREADS), 0, stream, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(latent_absorb_kernel, dim3(n_kv, (B + LT_ABS_SEQ - 1) / LT_ABS_SEQ), dim3(LT_ABS_THREADS), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_hg = (int)((n_q + LT_HEADS_PER_WG - 1) / LT_HEADS_PER_WG);
    hipLaunchKernelGGL(latent_split_kernel<false>, dim3(n_split, B, n_hg), dim3(LT_THREADS), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(latent_split_kernel<true>, dim3(n_split, B, n_hg), dim3(LT_THREADS), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(latent_combine_kernel, dim3(n_kv, B), dim3(LT_C), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdla
