// prefill_gfx950.hip -- fused GDLA attention core for prefill on gfx950.
//
// One workgroup computes one (sequence b, KV head j, tile of 64 query
// tokens) item for all five query heads of the group -- signal heads
// 4j..4j+3 and noise head j share the KV head's K and V (aitrends.kr, GDLA
// paragraph: both paths share one KV head; metalmedia Table 1: 64 signal +
// 16 noise heads over 16 KV heads).  Steps, all in this one kernel:
//   1. band limits: the key tiles a query tile can see -- 0..t for a full
//      causal layer, t-W+1..t for a sliding-window layer (aitrends.kr,
//      context-parallel paragraph: full attention costs Theta(L^2), sliding
//      window Theta(LW)); tiles outside the band are never loaded;
//   2. K and V tiles stream HBM -> LDS with direct (register-free) 16-byte
//      loads into a ring of three tile slots, two tiles ahead, shared by the
//      4 waves and all 5 heads; V stays row-major and the P*V operand is read
//      with the gfx950 LDS transpose read (ds_read_b64_tr_b16);
//   3. S^T = K Q^T on the matrix cores (bf16 in, fp32 out); the causal /
//      window mask enters as the products' initial value (0 or -inf) on the
//      slices that straddle the band edge only;
//   4. online softmax in base 2 with the scale folded in.  Each row's
//      reference maximum is fixed before the key loop by the visible keys of
//      the row's own 16-key block (the row maximum is not tracked after that),
//      so the accumulators are never rescaled inside the loop and stay in the
//      matrix-core register file, and every slice runs the same straight-line
//      code.
//      Row sums are taken over the same bf16-rounded weights that enter P*V.
//      If a row's sum ends a query tile far above its reference range (logits
//      that grew by more than ~40 natural units; rare), the workgroup redoes
//      that query tile: a scores-only pass finds the exact row maxima, then
//      the normal pass runs with those as references;
//   5. O^T += V^T P^T on the matrix cores;
//   6. epilogue in registers: H = O / l, D = H_S - lambda * H_N (each noise
//      row repeated to its 4 signal heads), out = gate * D, rounded to bf16
//      (aitrends.kr, GDLA paragraph: D_t = H_S,t - lambda_t (.) Repeat_g(H_N,t)
//      followed by the element-wise gate).
//
// Wave w of the workgroup owns query tokens t0+16w .. t0+16w+15 for all five
// heads: 5 query blocks of 16 in the N dimension of the 16x16x32 MFMA, so the
// noise row a signal row needs sits in the same lane.
#include "gdla_device.h"
#include "gdla_launch.h"

#include <algorithm>
#include <atomic>

namespace gdla {

constexpr int PF_BM = 64;             // query tokens per workgroup
constexpr int PF_BN = 64;             // keys per LDS tile
constexpr int PF_THREADS = 256;       // 4 waves
constexpr int KK_STEPS = D_QK / 32;   // MFMA k-steps over the query-key dim
// LDS rows carry a 32-byte pad so that the fragment reads of 16 consecutive
// rows spread over all banks (K: 416-byte rows, V: 288-byte rows).  Measured
// on gfx950: a 16-byte pad still leaves half the LDS cycles in bank conflicts
// for both the 16-byte K reads and the transposing V reads; 32 bytes removes them.
constexpr int ROW_PAD_CHUNKS = 2;
constexpr int KS_CHUNKS = D_QK / 8 + ROW_PAD_CHUNKS;   // 26 chunks of 16 bytes per K row
constexpr int VS_CHUNKS = D_V / 8 + ROW_PAD_CHUNKS;    // 18 chunks per V row
constexpr int KS_ROW = KS_CHUNKS * 8;              // bf16 per K row in LDS
constexpr int VS_ROW = VS_CHUNKS * 8;              // bf16 per V row in LDS
// A tile is copied by wave-wide instructions that each cover whole rows: two
// K rows (52 of 64 lanes) or three V rows (54 lanes), so a lane's row and
// chunk within the instruction never change and pad chunks are skipped.
constexpr int K_ROWS_PER_COPY = 2;
constexpr int V_ROWS_PER_COPY = 3;
constexpr int K_TILE_COPIES = PF_BN / K_ROWS_PER_COPY;                          // 32
constexpr int V_TILE_COPIES = (PF_BN + V_ROWS_PER_COPY - 1) / V_ROWS_PER_COPY;  // 22
static_assert(K_ROWS_PER_COPY * KS_CHUNKS <= 64 && V_ROWS_PER_COPY * VS_CHUNKS <= 64, "rows per copy");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

typedef __attribute__((address_space(3))) void lds_void_t;

// Buffer resource over `bytes` bytes from `base` (raw, no stride): reads at
// byte offsets >= bytes return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// This lane's index, read afresh: values derived from it are formed where they
// are used rather than held in registers across the key loop.
__device__ __forceinline__ int lane_now() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
// Buffer reads and writes at a byte offset: an offset at or past the
// resource's size reads zeros and drops the write.  The query, gate, lambda
// and output resources start at the first valid row of a query tile, so a row
// before it has a negative offset (far past the size as unsigned; a lane's
// column offset stays within its row, so the sum never wraps) and a row past
// the last valid one lies past the size.
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
}
__device__ __forceinline__ u32x2 bld8(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
}
// The output store is non-temporal (cache policy nt): the output is written
// once and never read back here, and keeping it out of the caches' normal
// replacement measured faster on full-causal layers (4K: 0.445 -> 0.437 ms)
// and within 1 % on a 128-token window.
__device__ __forceinline__ void bst16(__amdgpu_buffer_rsrc_t rs, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 2);
}

// One 16-byte buffer -> LDS copy per lane; lane l writes lds_base + 16*l.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t byte_off, __bf16 *lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)lds_base, 16, byte_off, 0, 0, 0);
}

// Wait until this wave's outstanding vector-memory loads (including the
// direct-to-LDS copies) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposing LDS read: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte words fetched by lanes 4e + i/4 (e = 0..3).
__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p));
}

struct PrefillParams {
    const __bf16 *qs, *qn, *k, *v, *lam, *gate;
    __bf16 *out;
    __bf16 *hs, *hn;                  // saving mode: the per-head outputs H_S [rows][n_sig][D_V], H_N [rows][n_kv][D_V]
    float *lse;                       // saving mode: log2 of each head's softmax sum, [rows][n_sig + n_kv]
    int B, n_kv, window;
    int Tq;                           // query rows per sequence (positions P .. P+Tq-1)
    int P;                            // keys before the first query (a prefix already in K/V)
    float scale_log2;                 // softmax scale * log2(e)
    int n_qt;                         // query tiles per sequence
    int run_len;                      // query tiles per work item
    int n_runs;                       // work items per sequence and KV head
};

// Work item = (head instance hi = b*n_kv + j, a run of consecutive query
// tiles).  The kernel is persistent: one workgroup per CU walks a fixed list
// of items, so that the next item's queries and first K/V tiles load while the
// current item's epilogue runs, and no CU waits for a new workgroup.  Items
// are ranked by cost (full causal: the last query tiles, the heaviest, first)
// and dealt in snake order -- round r goes to the workgroups in ascending
// order for even r and descending for odd r -- which evens out the work per
// CU.  When the head instances split evenly over the 8 XCDs, the workgroups of
// one XCD (blockIdx % 8: workgroups are spread over the XCDs in turn) deal
// only the items of that XCD's heads, so a head's K/V stays in one L2.
struct WorkList {
    bool by_xcd;
    int xcd;          // heads of this list: hi = 8m + xcd (by_xcd), else all
    int l, n_l;       // this workgroup's place among the n_l sharing the list
    int heads;        // head instances in the list
    int n_items;      // items in the list
};

__device__ __forceinline__ bool work_item(const WorkList &w, int round, int n_runs, int run_len,
                                          bool causal, int &hi, int &qt_first) {
    const int li = round * w.n_l + ((round & 1) ? w.n_l - 1 - w.l : w.l);
    if (li >= w.n_items) return false;
    const int rank = li / w.heads, m = li % w.heads;
    hi = w.by_xcd ? 8 * m + w.xcd : m;
    qt_first = (causal ? n_runs - 1 - rank : rank) * run_len;
    return true;
}

// PREFIX: queries start after a prefix of keys (P > 0); the P = 0 instance
// folds the position offsets away.
// TRAIN: also save what the backward needs (the per-head outputs and the
// log2-sum-exp of every head's row, reference included).
template <bool PREFIX, bool TRAIN>
__global__ __launch_bounds__(PF_THREADS, 1) void prefill_kernel(PrefillParams p) {
    // ring of three K and three V tile slots: key tile t lives in slot t % 3
    __shared__ __attribute__((aligned(16))) __bf16 Kring[3][PF_BN * KS_ROW];
    __shared__ __attribute__((aligned(16))) __bf16 Vring[3][PF_BN * VS_ROW];
    __shared__ int restart_flag[2];   // restart requests, by parity of the query tiles done

    // positions: query row i sits at P + i; every position < T holds a key.
    // Query tiles start at q0 = P rounded down to 64 so that they line up with
    // the key tiles; rows outside P .. T-1 are computed but never stored.
    const int Tq = p.Tq, P = PREFIX ? p.P : 0, q0 = P / PF_BM * PF_BM, T = P + Tq;
    const int n_kv = p.n_kv, window = p.window;
    const int n_sig = n_kv * GROUP;
    const int n_hi = p.B * n_kv;
    WorkList wl;
    wl.by_xcd = (n_hi & 7) == 0 && (gridDim.x & 7) == 0;
    wl.xcd = wl.by_xcd ? blockIdx.x & 7 : 0;
    wl.l = wl.by_xcd ? blockIdx.x >> 3 : blockIdx.x;
    wl.n_l = wl.by_xcd ? gridDim.x >> 3 : gridDim.x;
    wl.heads = wl.by_xcd ? n_hi >> 3 : n_hi;
    wl.n_items = p.n_runs * wl.heads;
    const bool causal = window == 0;
    int round = 0, hi, qt_first;
    if (!work_item(wl, round, p.n_runs, p.run_len, causal, hi, qt_first)) return;
    int b = hi / n_kv, j = hi % n_kv;
    int qt_end = min(qt_first + p.run_len, p.n_qt);           // one past the run's last query tile

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    long kseq0 = (long)b * T;         // first K/V row of sequence b
    long qseq0 = (long)b * Tq;        // first query (and gate / lambda / out) row of sequence b

    // key tiles a query tile sees: 0..t for a full causal layer, t-W+1..t with a window
    auto tile_lo = [&](int qt) { return window > 0 ? max(0, q0 + qt * PF_BM - window + 1) / PF_BN : 0; };
    auto tile_hi = [&](int qt) { return (min(q0 + qt * PF_BM + PF_BM, T) - 1) / PF_BN; };

    // ---- direct HBM -> LDS copy of key tile kt through buffer resources that
    // cover this sequence's rows of KV head j: rows past the sequence end read
    // as zeros (those keys are always masked).  A lane's byte offset within a
    // copy is fixed; the tile and copy add a uniform offset.
    const uint32_t krow_b = (uint32_t)n_kv * D_QK * 2, vrow_b = (uint32_t)n_kv * D_V * 2;
    __amdgpu_buffer_rsrc_t k_rsrc, v_rsrc;
    auto set_rsrc = [&](long s0, int jj) {
        k_rsrc = make_rsrc(p.k + (s0 * n_kv + jj) * D_QK, (uint32_t)T * krow_b);
        v_rsrc = make_rsrc(p.v + (s0 * n_kv + jj) * D_V, (uint32_t)T * vrow_b);
    };
    set_rsrc(kseq0, j);
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int k_lr = lane / KS_CHUNKS, k_ch = lane % KS_CHUNKS;    // row within the copy, chunk
    const int v_lr = lane / VS_CHUNKS, v_ch = lane % VS_CHUNKS;
    const bool k_on = k_lr < K_ROWS_PER_COPY && k_ch < D_QK / 8;  // pad chunks are not copied
    const bool v_on = v_lr < V_ROWS_PER_COPY && v_ch < D_V / 8;
    const uint32_t k_lane = k_lr * krow_b + 16 * k_ch, v_lane = v_lr * vrow_b + 16 * v_ch;
    auto issue_tile = [&](int kt) {
        __bf16 *ks = Kring[kt % 3], *vs = Vring[kt % 3];
        const int kbase = kt * PF_BN;
#pragma unroll
        for (int c = 0; c < K_TILE_COPIES / 4; ++c) {
            const int row0 = K_ROWS_PER_COPY * (uwave + 4 * c);
            if (k_on) copy16_to_lds(k_rsrc, k_lane + (uint32_t)(kbase + row0) * krow_b, ks + row0 * KS_ROW);
        }
#pragma unroll
        for (int c = 0; c < (V_TILE_COPIES + 3) / 4; ++c) {
            const int row0 = V_ROWS_PER_COPY * (uwave + 4 * c);
            if (row0 < PF_BN && v_on && row0 + v_lr < PF_BN)
                copy16_to_lds(v_rsrc, v_lane + (uint32_t)(kbase + row0) * vrow_b, vs + row0 * VS_ROW);
        }
    };
    // Tile t may be copied into slot t % 3 once tile t-3 is no longer needed:
    // at most two tiles past the tile being computed and past the lowest tile
    // any later query tile of the run still reads.  A run's query tiles see at
    // most three key tiles each (the host uses runs only when that holds).
    int run_last_tile = tile_hi(qt_end - 1);
    int next_copy;                    // lowest tile not yet copied
    auto start_ring = [&](int qt) {   // first two tiles of a query tile, nothing in flight
        next_copy = tile_lo(qt);
        issue_tile(next_copy++);
        if (next_copy <= tile_hi(qt)) issue_tile(next_copy++);
    };
    start_ring(qt_first);

    // ---- per-query-tile state, reset for every query tile of the run
    int t0 = q0 + qt_first * PF_BM;
    int tw = t0 + 16 * wave;          // first query token of this wave
    int tq = tw + r;                  // query token of this lane
    bf16x8 qf[HEADS][KK_STEPS];
    // B operand fragments of query tile qt of the sequence whose query rows
    // start at s0, KV head jj: lane holds Q[tq][32kk + 8g .. +7]
    // Rows of the tile outside P .. T-1 read zeros (outside the resources), and
    // qt < 0 (no next tile) reads nothing: the loads are issued unconditionally.
    auto load_q = [&](int qt, long s0, int jj) {
        const int tf = q0 + qt * PF_BM;                       // position of the tile's first row
        const int lo = PREFIX ? max(tf, P) : tf, end = min(tf + PF_BM, T);
        const long r0 = s0 + (PREFIX ? lo - P : lo);          // query row of position lo
        const int ln = lane_now();
        const int dt = tf + 16 * uwave + (ln & 15) - lo;      // row of this lane from the first valid one
        const uint32_t nrows = qt < 0 ? 0u : (uint32_t)max(0, end - lo);
        const auto qs_rs = make_rsrc(p.qs + (r0 * n_sig + GROUP * jj) * D_QK, nrows * (uint32_t)(n_sig * D_QK * 2));
        const auto qn_rs = make_rsrc(p.qn + (r0 * n_kv + jj) * D_QK, nrows * (uint32_t)(n_kv * D_QK * 2));
        const uint32_t os = (uint32_t)dt * (uint32_t)(n_sig * D_QK * 2) + 16 * (ln >> 4);
        const uint32_t on = (uint32_t)dt * (uint32_t)(n_kv * D_QK * 2) + 16 * (ln >> 4);
#pragma unroll
        for (int kk = 0; kk < KK_STEPS; ++kk) {
#pragma unroll
            for (int h = 0; h < GROUP; ++h) qf[h][kk] = __builtin_bit_cast(bf16x8, bld16(qs_rs, os + h * D_QK * 2 + 64 * kk));
            qf[GROUP][kk] = __builtin_bit_cast(bf16x8, bld16(qn_rs, on + 64 * kk));
        }
    };
    load_q(qt_first, qseq0, j);

    // l_part[h]: this lane's part of each row sum, over the bf16-rounded
    // weights that also enter P*V (so numerator and denominator agree)
    float m_ref[HEADS], l_part[HEADS];
    f32x4 o[HEADS][D_V / 16];
    const float c_log2 = p.scale_log2;
    if (tid < 2) restart_flag[tid] = 0;
    int n_done = 0;                   // query tiles finished by the workgroup
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // Masking enters the scores through the products' initial value: 0 for a
    // visible (key, query) pair, -inf for a hidden one, so a hidden key's weight
    // is exp2(-inf) = 0 and no branch or select touches the scores.  bias[kb]
    // covers this lane's keys kb0 + 16 kb + 4g + e (e = 0..3) for its query tq.
    auto make_bias = [&](int kb0, f32x4 (&bias)[2]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = kb0 + 16 * (i >> 2) + 4 * g + (i & 3);
            const bool vis = key <= tq && (window == 0 || key > tq - window);
            bias[i >> 2][i & 3] = vis ? 0.f : -INFINITY;
        }
    };

    // ---- the reference of each row (log2 units): the largest score over the
    // visible keys of the row's own 16-key block (key tq is always visible).
    // K rows tw .. tw+15 come straight from global memory as A fragments.
    auto ref_pass = [&]() {
        // (rows past the sequence end read zeros: their keys are visible only
        // to rows past the end, which are never stored)
        const int ln = lane_now();
        const uint32_t koff = (uint32_t)(tw + (ln & 15)) * krow_b + 16 * (ln >> 4);
        bf16x8 kf[KK_STEPS];
#pragma unroll
        for (int kk = 0; kk < KK_STEPS; ++kk) kf[kk] = __builtin_bit_cast(bf16x8, bld16(k_rsrc, koff + 64 * kk));
        f32x4 bias[2];
        make_bias(tw, bias);          // block 0 of a slice starting at key tw
        f32x4 sd[HEADS];
#pragma unroll
        for (int kk = 0; kk < KK_STEPS; ++kk)
#pragma unroll
            for (int h = 0; h < HEADS; ++h) sd[h] = mfma16(kf[kk], qf[h][kk], kk == 0 ? bias[0] : sd[h]);
#pragma unroll
        for (int h = 0; h < HEADS; ++h) {
            const float mx = fmaxf(fmaxf(sd[h][0], sd[h][1]), fmaxf(sd[h][2], sd[h][3]));
            m_ref[h] = group4_max(mx) * c_log2;
        }
    };

    // slice-level skips (wave-uniform): no valid query, all keys in the future,
    // all keys too old; and whether a slice needs masking at all
    auto slice_skipped = [&](int kb0) {
        return tw >= T || (PREFIX && tw + 15 < P) || kb0 > tw + 15 ||
               (window > 0 && kb0 + 31 < tw - window + 1);
    };
    auto slice_masked = [&](int kb0) {
        return (kb0 + 31 > tw) || (window > 0 && kb0 < tw + 16 - window);
    };

    // ---- one 32-key slice: S^T = K Q^T, weights against the fixed references,
    // O^T += V^T P^T.  Straight-line code (one basic block from the first K read
    // to the last product), so that the exponentials of block 0 overlap the
    // products of block 1 and those of block 1 the P*V products.
    auto slice = [&](int sub, const __bf16 *ks, const __bf16 *vs, const f32x4 (&bias)[2]) {
        const __bf16 *krd = ks + (32 * sub + r) * KS_ROW + 8 * g;
        f32x4 s[HEADS][2];
        uint32_t pw[HEADS][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const __bf16 *kr = krd + 16 * kb * KS_ROW;
            bf16x8 kf[KK_STEPS];
#pragma unroll
            for (int kk = 0; kk < KK_STEPS; ++kk) kf[kk] = *reinterpret_cast<const bf16x8 *>(kr + 32 * kk);
#pragma unroll
            for (int kk = 0; kk < KK_STEPS; ++kk)
#pragma unroll
                for (int h = 0; h < HEADS; ++h) s[h][kb] = mfma16(kf[kk], qf[h][kk], kk == 0 ? bias[kb] : s[h][kb]);
#pragma unroll
            for (int h = 0; h < HEADS; ++h) {
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) pv[e] = fast_exp2(fmaf(s[h][kb][e], c_log2, -m_ref[h]));
                pw[h][2 * kb] = pack_bf16x2(pv[0], pv[1]);
                pw[h][2 * kb + 1] = pack_bf16x2(pv[2], pv[3]);
            }
        }
        bf16x8 pb[HEADS];
#pragma unroll
        for (int h = 0; h < HEADS; ++h) {
            const u32x4 w = {pw[h][0], pw[h][1], pw[h][2], pw[h][3]};
            pb[h] = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int i = 0; i < 4; ++i) l_part[h] = sum_bf16x2(pw[h][i], l_part[h]);
        }
        // O^T += V^T P^T.  The A operand (16 columns x 32 keys) comes from two
        // transposing reads of row-major V: lane (r, g) receives V[4g + e][col]
        // and V[16 + 4g + e][col], e = 0..3 -- the keys its P^T fragment holds
        // in k-slots 8g..8g+7 -- for column col = 32c + 8(r/4) + 4s + r%4 of
        // block cb = 2c + s.  With that order the output lane (r, g) holds
        // columns 32c + 8g .. 32c + 8g + 7 of blocks 2c and 2c+1: 16 contiguous
        // bytes for the gate loads and output stores.
        const __bf16 *vrd = vs + (32 * sub + 4 * g + (r >> 2)) * VS_ROW + 8 * (r & 3);
        auto vfrag = [&](int cb) {
            const int cc = 32 * (cb >> 1) + 4 * (cb & 1);
            const s16x4 lo = lds_read_tr16(vrd + cc);
            const s16x4 hi4 = lds_read_tr16(vrd + 16 * VS_ROW + cc);
            const s16x4 v8[2] = {lo, hi4};
            return __builtin_bit_cast(bf16x8, v8);
        };
        bf16x8 va = vfrag(0);
#pragma unroll
        for (int cb = 0; cb < D_V / 16; ++cb) {
            bf16x8 nv = va;
            if (cb + 1 < D_V / 16) nv = vfrag(cb + 1);
#pragma unroll
            for (int h = 0; h < HEADS; ++h) o[h][cb] = mfma16(va, pb[h], o[h][cb]);
            va = nv;
        }
    };

    // scores only (the redo's first pass): exact row maxima over the visible keys
    auto max_slice = [&](int sub, const __bf16 *ks, const f32x4 (&bias)[2]) {
        const __bf16 *krd = ks + (32 * sub + r) * KS_ROW + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const __bf16 *kr = krd + 16 * kb * KS_ROW;
            bf16x8 kf[KK_STEPS];
#pragma unroll
            for (int kk = 0; kk < KK_STEPS; ++kk) kf[kk] = *reinterpret_cast<const bf16x8 *>(kr + 32 * kk);
            f32x4 sb[HEADS];
#pragma unroll
            for (int kk = 0; kk < KK_STEPS; ++kk)
#pragma unroll
                for (int h = 0; h < HEADS; ++h) sb[h] = mfma16(kf[kk], qf[h][kk], kk == 0 ? bias[kb] : sb[h]);
#pragma unroll
            for (int h = 0; h < HEADS; ++h) {
                const float mx = fmaxf(fmaxf(sb[h][0], sb[h][1]), fmaxf(sb[h][2], sb[h][3]));
                m_ref[h] = fmaxf(m_ref[h], group4_max(mx) * c_log2);
            }
        }
    };

    // ---- the key tiles of query tile qt.  MODE 0: the normal pass (checks the
    // row sums at the end), 1: scores only, 2: the normal pass after it (the
    // references are exact maxima: every weight <= 1).  Before each barrier a
    // wave drains its older copies and all LDS traffic but may leave its newest
    // batch (13 or 14 copies) in flight when the tile computed next is older
    // than it.  The barrier is the bare s_barrier: a workgroup fence would also
    // drain the newest copies.  Returns whether any wave asked for the redo.
    auto run_tiles = [&](int qt, int kt_lo, int kt_hi, int next_lo, const int mode) {
        bool wave_restart = false;
        for (int kt = kt_lo; kt <= kt_hi; ++kt) {
            const __bf16 *ks = Kring[kt % 3], *vs = Vring[kt % 3];
            // kept rolled: unrolling lets the scheduler overlap two slices,
            // which doubles the live scores and spills
#pragma unroll 1
            for (int sub = 0; sub < 2; ++sub) {
                const int kb0 = kt * PF_BN + 32 * sub;
                if (slice_skipped(kb0)) continue;
                f32x4 bias[2];
                if (slice_masked(kb0)) make_bias(kb0, bias);
                else bias[0] = bias[1] = zero4;
                if (mode == 1) max_slice(sub, ks, bias);
                else slice(sub, ks, vs, bias);
            }
            const bool last = kt == kt_hi;
            if (last && mode == 0 && (!PREFIX || tq >= P) && tq < T) {
#pragma unroll
                for (int h = 0; h < HEADS; ++h) wave_restart |= !(l_part[h] <= RESTART_PART_SUM);
            }
            // the redo passes end where the normal pass ended: the same copies
            // for the query tile that follows
            const int nt = !last ? kt + 1 : (mode == 1 ? kt_lo : next_lo);   // tile computed next
            const int limit = min(min(kt, nt) + 2, mode == 1 ? kt_hi : run_last_tile);
            while (next_copy <= limit) issue_tile(next_copy++);
            if (last && mode == 0 && __any(wave_restart) && lane == 0) restart_flag[n_done & 1] = 1;
            if (next_copy - 1 > nt) __builtin_amdgcn_s_waitcnt(0x007D);   // vmcnt(13) lgkmcnt(0)
            else __builtin_amdgcn_s_waitcnt(0x0070);                      // vmcnt(0) lgkmcnt(0)
            asm volatile("" ::: "memory");                                // no compiler motion across
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        return mode == 0 && __builtin_amdgcn_readfirstlane(restart_flag[n_done & 1]) != 0;
    };

    wait_vmem();
    __syncthreads();
    for (;;) {                        // work items of this workgroup
    bool more_items = false;
    for (int qt = qt_first; qt < qt_end; ++qt) {
        t0 = q0 + qt * PF_BM;
        tw = t0 + 16 * wave;
        tq = tw + r;
        const int kt_lo = tile_lo(qt), kt_hi = tile_hi(qt);
        const int next_lo = qt + 1 < qt_end ? tile_lo(qt + 1) : 1 << 30;
#pragma unroll
        for (int h = 0; h < HEADS; ++h) {
            l_part[h] = 0.f;
#pragma unroll
            for (int cb = 0; cb < D_V / 16; ++cb) o[h][cb] = zero4;
        }
        // The weights are taken against the references of ref_pass.  If a
        // lane's part of a row sum ends above 2^62 (or is not finite), the
        // workgroup redoes the query tile in two passes: scores only, for the
        // exact row maxima, then the normal pass with those as references
        // (every weight <= 1, so no sum comes near 2^62).
        ref_pass();
        if (run_tiles(qt, kt_lo, kt_hi, next_lo, 0)) {
            wait_vmem();
            __syncthreads();                   // every wave has read the flag
            if (tid == 0) restart_flag[n_done & 1] = 0;
#pragma unroll
            for (int h = 0; h < HEADS; ++h) m_ref[h] = -INFINITY;
            start_ring(qt);
            wait_vmem();
            __syncthreads();
            run_tiles(qt, kt_lo, kt_hi, next_lo, 1);
#pragma unroll
            for (int h = 0; h < HEADS; ++h) {
                l_part[h] = 0.f;
#pragma unroll
                for (int cb = 0; cb < D_V / 16; ++cb) o[h][cb] = zero4;
            }
            wait_vmem();
            __syncthreads();
            start_ring(qt);
            wait_vmem();
            __syncthreads();
            run_tiles(qt, kt_lo, kt_hi, next_lo, 2);
        }
        ++n_done;

        // ---- epilogue: normalise, differential combine, gate, bf16 store.
        // Requested in this order: the first K/V tiles of what comes next, this
        // tile's gate and lambda, the next query tile's queries; then the math
        // and the stores.  No load or store depends on a branch, so the waits
        // the compiler places are exact (no spill reload or untaken path forces
        // a full drain).
        const bool row_ok = (!PREFIX || tq >= P) && tq < T;
        const long row = qseq0 + (row_ok ? (PREFIX ? tq - P : tq) : 0);     // saved outputs only
        // next query tile of the run, or the first of the next work item: every
        // wave is done with the ring, so that item's first K/V tiles are copied
        // now, behind this epilogue, as are its queries
        int n_b = b, n_j = j, n_qt = qt + 1;
        if (n_qt >= qt_end) {
            if (work_item(wl, round + 1, p.n_runs, p.run_len, causal, hi, n_qt)) {
                more_items = true;
                n_b = hi / n_kv;
                n_j = hi % n_kv;
                set_rsrc((long)n_b * T, n_j);
                run_last_tile = tile_hi(min(n_qt + p.run_len, p.n_qt) - 1);
                start_ring(n_qt);
            } else {
                n_qt = -1;
            }
        }
        // This tile's gate and lambda are requested after those copies and
        // before the queries, so that their first use waits for them alone.
        // Gate, lambda and out go through resources over the tile's valid rows:
        // the other rows read zeros and their writes are dropped, so the loads
        // and stores carry no branch.
        const int e_lo = PREFIX ? max(t0, P) : t0, e_hi = min(t0 + PF_BM, T);
        const long e_r0 = qseq0 + (PREFIX ? e_lo - P : e_lo);
        const uint32_t e_rows = (uint32_t)max(0, e_hi - e_lo);
        const auto g_rs = make_rsrc(p.gate + (e_r0 * n_sig + GROUP * j) * D_V, e_rows * (uint32_t)(n_sig * D_V * 2));
        const auto o_rs = make_rsrc(p.out + (e_r0 * n_sig + GROUP * j) * D_V, e_rows * (uint32_t)(n_sig * D_V * 2));
        const auto l_rs = make_rsrc(p.lam + e_r0 * n_sig + GROUP * j, e_rows * (uint32_t)(n_sig * 2));
        const int eln = lane_now();
        const int edt = tw + (eln & 15) - e_lo;               // row of this lane from the first valid one
        const uint32_t e_off = (uint32_t)edt * (uint32_t)(n_sig * D_V * 2) + 16 * (eln >> 4);
        u32x4 gw[GROUP][D_V / 32];
#pragma unroll
        for (int c = 0; c < D_V / 32; ++c)
#pragma unroll
            for (int h = 0; h < GROUP; ++h) gw[h][c] = bld16(g_rs, e_off + h * D_V * 2 + 64 * c);
        const u32x2 lw = bld8(l_rs, (uint32_t)edt * (uint32_t)(n_sig * 2));
        load_q(n_qt, (long)n_b * Tq, n_j);
        // (an opaque copy: the store offsets are then formed next to the
        // stores, as immediates on one register)
        uint32_t so = e_off;
        asm volatile("" : "+v"(so));

        float inv[HEADS];
#pragma unroll
        for (int h = 0; h < HEADS; ++h) inv[h] = 1.f / group4_sum(l_part[h]);
        {
            const float lam[GROUP] = {bf16_lo(lw[0]), bf16_hi(lw[0]), bf16_lo(lw[1]), bf16_hi(lw[1])};
#pragma unroll
            for (int c = 0; c < D_V / 32; ++c) {
                // columns 32c + 8g .. +7: blocks 2c (first four) and 2c + 1
                const int col = 32 * c + 8 * g;
                float hn[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) hn[e] = o[GROUP][2 * c + e / 4][e % 4] * inv[GROUP];
#pragma unroll
                for (int h = 0; h < GROUP; ++h) {
                    float y[8], hs[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t gword = gw[h][c][e / 2];
                        const float gv = (e & 1) ? bf16_hi(gword) : bf16_lo(gword);
                        // H_S and H_N are formed the same way, so identical queries with
                        // lambda = 1 give exactly 0
                        hs[e] = o[h][2 * c + e / 4][e % 4] * inv[h];
                        y[e] = gv * fmaf(-lam[h], hn[e], hs[e]);
                    }
                    bst16(o_rs, so + h * D_V * 2 + 64 * c,
                          u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                pack_bf16x2(y[6], y[7])});
                    if constexpr (TRAIN) if (row_ok)
                        *reinterpret_cast<u32x4 *>(p.hs + (row * n_sig + GROUP * j + h) * D_V + col) =
                            u32x4{pack_bf16x2(hs[0], hs[1]), pack_bf16x2(hs[2], hs[3]), pack_bf16x2(hs[4], hs[5]),
                                  pack_bf16x2(hs[6], hs[7])};
                }
                if constexpr (TRAIN) if (row_ok)
                    *reinterpret_cast<u32x4 *>(p.hn + (row * n_kv + j) * D_V + col) =
                        u32x4{pack_bf16x2(hn[0], hn[1]), pack_bf16x2(hn[2], hn[3]), pack_bf16x2(hn[4], hn[5]),
                              pack_bf16x2(hn[6], hn[7])};
            }
            if constexpr (TRAIN) if (row_ok) {
                // the weights were exp2(score * scale * log2(e) - m_ref) with sum 1/inv
                if (g == 0) {
#pragma unroll
                    for (int h = 0; h < HEADS; ++h) {
                        const float m = m_ref[h] == -INFINITY ? 0.f : m_ref[h];
                        const int col = h < GROUP ? GROUP * j + h : n_sig + j;
                        p.lse[row * (n_sig + n_kv) + col] = m - __log2f(inv[h]);
                    }
                }
            }
        }
        if (more_items) {
            b = n_b;
            j = n_j;
            kseq0 = (long)b * T;
            qseq0 = (long)b * Tq;
            qt_first = n_qt;
        }
    }
    if (!more_items) break;
    ++round;
    qt_end = min(qt_first + p.run_len, p.n_qt);
    // the next item's first tiles and queries have landed in every wave.
    // Without the saved outputs a wave's last 16 memory operations are the
    // output stores, which need not complete first: vmcnt(16).  The barrier is
    // the bare s_barrier (a workgroup fence would wait for the stores too).
    static_assert(GROUP * D_V / 32 == 16, "output stores per wave");
    if constexpr (TRAIN) wait_vmem();
    else __builtin_amdgcn_s_waitcnt(0x4F70);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    }
}

// Compute units of the current device (read once per device).
static int compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_prefill(const void *qs, const void *qn, const void *k, const void *v,
                          const void *lam, const void *gate, void *out, int B, int Tq, int P, int n_kv,
                          int window, float scale, hipStream_t stream, void *save_hs, void *save_hn,
                          float *save_lse) {
    PrefillParams p;
    p.hs = static_cast<__bf16 *>(save_hs);
    p.hn = static_cast<__bf16 *>(save_hn);
    p.lse = save_lse;
    p.qs = static_cast<const __bf16 *>(qs);
    p.qn = static_cast<const __bf16 *>(qn);
    p.k = static_cast<const __bf16 *>(k);
    p.v = static_cast<const __bf16 *>(v);
    p.lam = static_cast<const __bf16 *>(lam);
    p.gate = static_cast<const __bf16 *>(gate);
    p.out = static_cast<__bf16 *>(out);
    p.B = B;
    p.Tq = Tq;
    p.P = P;
    p.n_kv = n_kv;
    p.window = window >= P + Tq ? 0 : window;  // a window covering the sequence is full causal
    p.scale_log2 = scale * LOG2E;
    p.n_qt = (P % PF_BM + Tq + PF_BM - 1) / PF_BM;
    // Sliding windows of up to 2*PF_BN+1 keys touch at most three key tiles per
    // query tile, so a workgroup can walk a run of consecutive query tiles and
    // copy one new K/V tile per query tile; runs are sized for about two per CU.
    const int n_cu = compute_units();
    p.run_len = 1;
    if (p.window > 0 && p.window <= 2 * PF_BN + 1) {
        const long tiles = (long)B * n_kv * p.n_qt;
        p.run_len = (int)std::max(1L, std::min((long)p.n_qt, (tiles + 2L * n_cu - 1) / (2L * n_cu)));
    }
    p.n_runs = (p.n_qt + p.run_len - 1) / p.run_len;
    // one persistent workgroup per CU (at most one fits: LDS and registers)
    const long items = (long)B * n_kv * p.n_runs;
    const long blocks = std::min(items, (long)n_cu);
    if (save_hs)        // the saving mode (a full prefill only)
        hipLaunchKernelGGL((prefill_kernel<false, true>), dim3((unsigned)blocks), dim3(PF_THREADS), 0, stream, p);
    else if (P > 0)
        hipLaunchKernelGGL((prefill_kernel<true, false>), dim3((unsigned)blocks), dim3(PF_THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<false, false>), dim3((unsigned)blocks), dim3(PF_THREADS), 0, stream, p);
    return hipGetLastError();
}

long prefill_grid_blocks(int B, int Tq, int P, int n_kv) {
    return (long)B * n_kv * ((P % PF_BM + (long)Tq + PF_BM - 1) / PF_BM);
}

}  // namespace gdla
