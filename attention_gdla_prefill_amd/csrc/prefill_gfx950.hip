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
//      8 waves and all 5 heads; V stays row-major and the P*V operand is read
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
//   6. epilogue: H = O / l, D = H_S - lambda * H_N (each noise row repeated
//      to its 4 signal heads), out = gate * D, rounded to bf16
//      (aitrends.kr, GDLA paragraph: D_t = H_S,t - lambda_t (.) Repeat_g(H_N,t)
//      followed by the element-wise gate).
//
// Two waves per SIMD.  A workgroup of 8 waves takes the tile of 64 query
// tokens; the 16 tokens of SIMD s (s = 0..3) are shared by its two waves:
//   wave s     ("A"): heads 0, 1 and the noise head (three 16-row MFMA blocks),
//   wave s + 4 ("B"): heads 2 and 3 (two blocks).
// One wave's exponentials then run while the other wave's products keep the
// matrix core busy.  A single wave holding all five heads (Q and the output
// accumulators alone take 280 of its 512 registers) has to interleave both
// itself, and the softmax of a slice's second key block waits on nothing but
// the products that follow it: that layout measured 433 ms at T = 131072
// against 365 ms for this one when it came in (on the same box).  Each wave needs at most 256 registers, so two
// fit on a SIMD.  In the epilogue wave A hands the normalised noise-head
// output H_N of its 16 tokens to wave B through LDS (lane to lane: both waves
// hold the same tokens and columns in the same lanes), in two halves of 64
// columns; each wave then forms the outputs of its two signal heads.
#include "gdla_device.h"
#include "gdla_launch.h"

#include <algorithm>
#include <atomic>
#include <cstdlib>

namespace gdla {

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

namespace pf {

constexpr int BM = 64;                 // query tokens per workgroup
constexpr int BN = 64;                 // keys per LDS tile
constexpr int THREADS = 512;           // 8 waves
constexpr int WAVES = THREADS / 64;
constexpr int KK = D_QK / 32;          // MFMA k-steps over the query-key dim
// LDS rows carry a 32-byte pad so that fragment reads of 16 consecutive rows
// spread over all banks (K: 416-byte rows, V: 288-byte rows).
constexpr int KS_CHUNKS = D_QK / 8 + 2;
constexpr int VS_CHUNKS = D_V / 8 + 2;
constexpr int KS_ROW = KS_CHUNKS * 8;
constexpr int VS_ROW = VS_CHUNKS * 8;
// A tile is copied by wave-wide instructions that each cover whole rows: two
// K rows (52 of 64 lanes) or three V rows (54 lanes).
constexpr int K_ROWS_PER_COPY = 2;
constexpr int V_ROWS_PER_COPY = 3;
constexpr int K_TILE_COPIES = BN / K_ROWS_PER_COPY;                          // 32: 4 per wave
constexpr int V_TILE_COPIES = (BN + V_ROWS_PER_COPY - 1) / V_ROWS_PER_COPY;  // 22: 3 or 2 per wave
constexpr int K_COPIES_PER_WAVE = K_TILE_COPIES / WAVES;
constexpr int V_COPIES_PER_WAVE = (V_TILE_COPIES + WAVES - 1) / WAVES;
static_assert(K_TILE_COPIES % WAVES == 0, "K copies split evenly over the waves");
static_assert(K_ROWS_PER_COPY * KS_CHUNKS <= 64 && V_ROWS_PER_COPY * VS_CHUNKS <= 64, "rows per copy");
// Waves 0 .. V_FULL_WAVES-1 issue V_COPIES_PER_WAVE copies of a tile, the others one fewer.
constexpr int V_FULL_WAVES = V_TILE_COPIES - WAVES * (V_COPIES_PER_WAVE - 1);   // 6
// H_N handed from wave A to wave B: [SIMD][lane][16 floats] per half
constexpr int XCH_FLOATS = 16;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ int lane_now() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
// Buffer reads and writes at a byte offset: an offset at or past the
// resource's size reads zeros and drops the write (rows outside a tile's
// valid range, with the resources starting at the first valid row).
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
}
__device__ __forceinline__ u32x2 bld8(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
}
// non-temporal output store (written once, never read back here)
__device__ __forceinline__ void bst16(__amdgpu_buffer_rsrc_t rs, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 2);
}
// One 16-byte buffer -> LDS copy per lane: lane l writes lds_addr + 16*l (the
// LDS address goes to M0).  Written as a statement the compiler does not model
// as an LDS write: otherwise it waits for every vector memory operation in
// flight before the next LDS read (the first K read of every slice), which
// drains the copies issued two tiles ahead and any other load in flight.  The
// kernel orders the copies against the reads itself: a wait for the wave's
// older copies and a barrier before a tile is read, and a slot is refilled
// only after the barrier that ends its last reader.  The nop is the wait state
// an LDS-DMA load needs after M0 is written.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 copy_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}
__device__ __forceinline__ void copy16_to_lds(const i32x4 &rsrc, uint32_t byte_off, uint32_t lds_addr) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(byte_off), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr_of(const __bf16 *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) __bf16 *)p;
}
// The same copy through the compiler's LDS-DMA builtin, which it does model as
// an LDS write (and so drains every vector memory operation in flight before
// the next LDS read).  Full-causal launches use this form: their workgroups,
// held back at every slice until the newest copies land, stay closer together
// on the key tiles they stream and share them in the L2 (the other form ran
// as fast there but fetched 2.6x more from beyond the L2 at T = 131072);
// sliding-window runs use the statement above (2.5 % faster).
__device__ __forceinline__ void copy16_to_lds_tracked(__amdgpu_buffer_rsrc_t rsrc, uint32_t byte_off, __bf16 *lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)lds_base, 16, byte_off, 0, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p));
}
// bare workgroup barrier (no fence: a fence would also drain copies in flight)
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// barrier after this wave's LDS accesses have completed (lgkmcnt(0)); copies
// and stores in flight stay in flight
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    bare_barrier();
}

// Work item = (head instance hi = b*n_kv + j, a run of consecutive query
// tiles).  The kernel is persistent: one workgroup per CU walks a fixed list
// of items, so that the next item's queries and first K/V tiles load while the
// current item's epilogue runs.  The list is head by head; within a head the
// items are ranked by cost (full causal: the last query tiles, the heaviest,
// first) and the list is dealt in snake order -- round r goes to the
// workgroups in ascending order for even r and descending for odd r.  When the
// head instances split evenly over the 8 XCDs, the workgroups of one XCD
// (blockIdx % 8) deal only the items of that XCD's heads, one head after the
// other, so the K/V tiles the XCD's workgroups stream at a time are those of
// one head, shared in that XCD's L2.
struct WorkList {
    bool by_xcd;
    int xcd, l, n_l, heads, n_items;
};

__device__ __forceinline__ bool work_item(const WorkList &w, int round, int n_runs, int run_len, bool causal,
                                          int &hi, int &qt_first) {
    const int li = round * w.n_l + ((round & 1) ? w.n_l - 1 - w.l : w.l);
    if (li >= w.n_items) return false;
    const int rank = li % n_runs, m = li / n_runs;
    hi = w.by_xcd ? 8 * m + w.xcd : m;
    qt_first = (causal ? n_runs - 1 - rank : rank) * run_len;
    return true;
}

// The heads of a wave: A = {0, 1, noise}, B = {2, 3}.  Head index 4 is the
// noise head.
template <int ROLE> struct Role;
template <> struct Role<0> {
    static constexpr int NH = 3;
    static constexpr int head(int i) { return i == 2 ? GROUP : i; }
    static constexpr int NOUT = 2;                   // signal heads it outputs: 0, 1
    static constexpr int out_head(int i) { return i; }
};
template <> struct Role<1> {
    static constexpr int NH = 2;
    static constexpr int head(int i) { return 2 + i; }
    static constexpr int NOUT = 2;                   // signal heads 2, 3
    static constexpr int out_head(int i) { return 2 + i; }
};

// LDS of a workgroup: the K and V ring, H_N handed from wave A to wave B
// ([4 SIMDs][64 lanes][XCH_FLOATS]), restart requests by parity of the query
// tiles done
typedef __bf16 KRing[3][BN * KS_ROW];
typedef __bf16 VRing[3][BN * VS_ROW];

template <bool PREFIX, bool TRAIN, bool ASMC, int ROLE>
__device__ __forceinline__ void run(const PrefillParams &p, KRing &kring, VRing &vring, float *xch_base,
                                    int *restart_flag) {
    using R = Role<ROLE>;
    constexpr int NH = R::NH;
    const int Tq = p.Tq, P = PREFIX ? p.P : 0, q0 = P / BM * BM, T = P + Tq;
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
    int qt_end = min(qt_first + p.run_len, p.n_qt);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int sub = wave & 3;                                  // the SIMD's 16 tokens
    const int r = lane & 15, g = lane >> 4;
    long kseq0 = (long)b * T;
    long qseq0 = (long)b * Tq;

    auto tile_lo = [&](int qt) { return window > 0 ? max(0, q0 + qt * BM - window + 1) / BN : 0; };
    auto tile_hi = [&](int qt) { return (min(q0 + qt * BM + BM, T) - 1) / BN; };

    // ---- K/V tile copies, HBM -> LDS: wave w issues K copies w, w+8, w+16,
    // w+24 and V copies w, w+8 (and w+16 for w < 6)
    const uint32_t krow_b = (uint32_t)n_kv * D_QK * 2, vrow_b = (uint32_t)n_kv * D_V * 2;
    __amdgpu_buffer_rsrc_t k_rsrc, v_rsrc;  // the reference pass's global K reads; the tracked copies
    i32x4 kc_rsrc, vc_rsrc;                 // the statement copies
    auto set_rsrc = [&](long s0, int jj) {
        k_rsrc = make_rsrc(p.k + (s0 * n_kv + jj) * D_QK, (uint32_t)T * krow_b);
        if constexpr (ASMC) {
            kc_rsrc = copy_rsrc(p.k + (s0 * n_kv + jj) * D_QK, (uint32_t)T * krow_b);
            vc_rsrc = copy_rsrc(p.v + (s0 * n_kv + jj) * D_V, (uint32_t)T * vrow_b);
        } else {
            v_rsrc = make_rsrc(p.v + (s0 * n_kv + jj) * D_V, (uint32_t)T * vrow_b);
        }
    };
    set_rsrc(kseq0, j);
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int k_lr = lane / KS_CHUNKS, k_ch = lane % KS_CHUNKS;
    const int v_lr = lane / VS_CHUNKS, v_ch = lane % VS_CHUNKS;
    const bool k_on = k_lr < K_ROWS_PER_COPY && k_ch < D_QK / 8;
    const bool v_on = v_lr < V_ROWS_PER_COPY && v_ch < D_V / 8;
    const uint32_t k_lane = k_lr * krow_b + 16 * k_ch, v_lane = v_lr * vrow_b + 16 * v_ch;
    auto issue_tile = [&](int kt) {
        __bf16 *ks = kring[kt % 3], *vs = vring[kt % 3];
        const int kbase = kt * BN;
#pragma unroll
        for (int c = 0; c < K_COPIES_PER_WAVE; ++c) {
            const int row0 = K_ROWS_PER_COPY * (uwave + WAVES * c);
            if (k_on) {
                if constexpr (ASMC)
                    copy16_to_lds(kc_rsrc, k_lane + (uint32_t)(kbase + row0) * krow_b, lds_addr_of(ks + row0 * KS_ROW));
                else
                    copy16_to_lds_tracked(k_rsrc, k_lane + (uint32_t)(kbase + row0) * krow_b, ks + row0 * KS_ROW);
            }
        }
#pragma unroll
        for (int c = 0; c < V_COPIES_PER_WAVE; ++c) {
            const int row0 = V_ROWS_PER_COPY * (uwave + WAVES * c);
            if (row0 < BN && v_on && row0 + v_lr < BN)
            {
                if constexpr (ASMC)
                    copy16_to_lds(vc_rsrc, v_lane + (uint32_t)(kbase + row0) * vrow_b, lds_addr_of(vs + row0 * VS_ROW));
                else
                    copy16_to_lds_tracked(v_rsrc, v_lane + (uint32_t)(kbase + row0) * vrow_b, vs + row0 * VS_ROW);
            }
        }
    };
    // Wait for this wave's copies of all but its newest tile (which may stay
    // in flight): the count is the wave's copy instructions per tile.
    auto wait_all_but_newest = [&]() {
        if (uwave < V_FULL_WAVES) __builtin_amdgcn_s_waitcnt(0x0077);   // vmcnt(7) lgkmcnt(0)
        else __builtin_amdgcn_s_waitcnt(0x0076);                        // vmcnt(6) lgkmcnt(0)
    };
    static_assert(K_COPIES_PER_WAVE + V_COPIES_PER_WAVE == 7, "copies per wave and tile");
    int run_last_tile = tile_hi(qt_end - 1);
    int next_copy;
    auto start_ring = [&](int qt) {
        next_copy = tile_lo(qt);
        issue_tile(next_copy++);
        if (next_copy <= tile_hi(qt)) issue_tile(next_copy++);
    };
    start_ring(qt_first);

    int t0 = q0 + qt_first * BM;
    int tw = t0 + 16 * sub;
    int tq = tw + r;
    bf16x8 qf[NH][KK];
    // B operand fragments of this wave's heads for query tile qt
    auto load_q = [&](int qt, long s0, int jj) {
        const int tf = q0 + qt * BM;
        const int lo = PREFIX ? max(tf, P) : tf, end = min(tf + BM, T);
        const long r0 = s0 + (PREFIX ? lo - P : lo);
        const int ln = lane_now();
        const int dt = tf + 16 * (uwave & 3) + (ln & 15) - lo;
        const uint32_t nrows = qt < 0 ? 0u : (uint32_t)max(0, end - lo);
        const auto qs_rs = make_rsrc(p.qs + (r0 * n_sig + GROUP * jj) * D_QK, nrows * (uint32_t)(n_sig * D_QK * 2));
        const auto qn_rs = make_rsrc(p.qn + (r0 * n_kv + jj) * D_QK, nrows * (uint32_t)(n_kv * D_QK * 2));
        const uint32_t os = (uint32_t)dt * (uint32_t)(n_sig * D_QK * 2) + 16 * (ln >> 4);
        const uint32_t on = (uint32_t)dt * (uint32_t)(n_kv * D_QK * 2) + 16 * (ln >> 4);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const int gh = R::head(h);
                qf[h][kk] = __builtin_bit_cast(bf16x8, gh < GROUP ? bld16(qs_rs, os + gh * D_QK * 2 + 64 * kk)
                                                                  : bld16(qn_rs, on + 64 * kk));
            }
    };
    load_q(qt_first, qseq0, j);

    float m_ref[NH], l_part[NH];
    f32x4 o[NH][D_V / 16];
    const float c_log2 = p.scale_log2;
    if (tid < 2) restart_flag[tid] = 0;
    int n_done = 0;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    auto make_bias = [&](int kb0, f32x4 (&bias)[2]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = kb0 + 16 * (i >> 2) + 4 * g + (i & 3);
            const bool vis = key <= tq && (window == 0 || key > tq - window);
            bias[i >> 2][i & 3] = vis ? 0.f : -INFINITY;
        }
    };

    // the reference of each row: the largest score over the visible keys of
    // the row's own 16-key block, K rows tw .. tw+15 -- rows 16*sub .. of the
    // diagonal key tile kt_diag.  Every copy issued so far has landed and is
    // visible when a query tile starts, so while that tile is still in the
    // ring (a sliding window, the first query tiles) its rows come from LDS,
    // else from global memory.
    auto ref_pass = [&](int kt_diag) {
        bf16x8 kf[KK];
        if (kt_diag >= next_copy - 3 && kt_diag < next_copy) {
            const __bf16 *kr = kring[kt_diag % 3] + (tw - kt_diag * BN + r) * KS_ROW + 8 * g;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) kf[kk] = *reinterpret_cast<const bf16x8 *>(kr + 32 * kk);
        } else {
            const int ln = lane_now();
            const uint32_t koff = (uint32_t)(tw + (ln & 15)) * krow_b + 16 * (ln >> 4);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) kf[kk] = __builtin_bit_cast(bf16x8, bld16(k_rsrc, koff + 64 * kk));
        }
        f32x4 bias[2];
        make_bias(tw, bias);
        f32x4 sd[NH];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int h = 0; h < NH; ++h) sd[h] = mfma16(kf[kk], qf[h][kk], kk == 0 ? bias[0] : sd[h]);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const float mx = fmaxf(fmaxf(sd[h][0], sd[h][1]), fmaxf(sd[h][2], sd[h][3]));
            m_ref[h] = group4_max(mx) * c_log2;
        }
    };

    auto slice_skipped = [&](int kb0) {
        return tw >= T || (PREFIX && tw + 15 < P) || kb0 > tw + 15 || (window > 0 && kb0 + 31 < tw - window + 1);
    };
    auto slice_masked = [&](int kb0) { return (kb0 + 31 > tw) || (window > 0 && kb0 < tw + 16 - window); };

    // one 32-key slice for this wave's heads
    auto slice = [&](int s32, const __bf16 *ks, const __bf16 *vs, const f32x4 (&bias)[2]) {
        const __bf16 *krd = ks + (32 * s32 + r) * KS_ROW + 8 * g;
        uint32_t pw[NH][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const __bf16 *kr = krd + 16 * kb * KS_ROW;
            bf16x8 kf[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) kf[kk] = *reinterpret_cast<const bf16x8 *>(kr + 32 * kk);
            f32x4 s[NH];
            // While a wave issues a chain of matrix products it outranks the
            // other wave of its SIMD, whose softmax arithmetic then fills the
            // issue slots between them; when both waves reach their products
            // together one runs ahead, which moves the pair out of step.
            if constexpr (!TRAIN) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int h = 0; h < NH; ++h) s[h] = mfma16(kf[kk], qf[h][kk], kk == 0 ? bias[kb] : s[h]);
            if constexpr (!TRAIN) __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) pv[e] = fast_exp2(fmaf(s[h][e], c_log2, -m_ref[h]));
                pw[h][2 * kb] = pack_bf16x2(pv[0], pv[1]);
                pw[h][2 * kb + 1] = pack_bf16x2(pv[2], pv[3]);
            }
        }
        bf16x8 pb[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const u32x4 w = {pw[h][0], pw[h][1], pw[h][2], pw[h][3]};
            pb[h] = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int i = 0; i < 4; ++i) l_part[h] = sum_bf16x2(pw[h][i], l_part[h]);
        }
        // O^T += V^T P^T: lane (r, g) receives V[4g + e][col] and V[16 + 4g + e][col],
        // col = 32c + 8(r/4) + 4s + r%4 of block 2c + s
        const __bf16 *vrd = vs + (32 * s32 + 4 * g + (r >> 2)) * VS_ROW + 8 * (r & 3);
        if constexpr (!TRAIN) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int cb = 0; cb < D_V / 16; ++cb) {
            const int cc = 32 * (cb >> 1) + 4 * (cb & 1);
            const s16x4 v8[2] = {lds_read_tr16(vrd + cc), lds_read_tr16(vrd + 16 * VS_ROW + cc)};
            const bf16x8 va = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
            for (int h = 0; h < NH; ++h) o[h][cb] = mfma16(va, pb[h], o[h][cb]);
        }
        if constexpr (!TRAIN) __builtin_amdgcn_s_setprio(0);
    };

    auto max_slice = [&](int s32, const __bf16 *ks, const f32x4 (&bias)[2]) {
        const __bf16 *krd = ks + (32 * s32 + r) * KS_ROW + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const __bf16 *kr = krd + 16 * kb * KS_ROW;
            bf16x8 kf[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) kf[kk] = *reinterpret_cast<const bf16x8 *>(kr + 32 * kk);
            f32x4 sb[NH];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int h = 0; h < NH; ++h) sb[h] = mfma16(kf[kk], qf[h][kk], kk == 0 ? bias[kb] : sb[h]);
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const float mx = fmaxf(fmaxf(sb[h][0], sb[h][1]), fmaxf(sb[h][2], sb[h][3]));
                m_ref[h] = fmaxf(m_ref[h], group4_max(mx) * c_log2);
            }
        }
    };

    // the key tiles of query tile qt.  MODE 0: normal pass, 1: scores only,
    // 2: the normal pass after it.  Returns whether any wave asked for the redo.
    auto run_tiles = [&](int qt, int kt_lo, int kt_hi, int next_lo, const int mode) {
        bool wave_restart = false;
        for (int kt = kt_lo; kt <= kt_hi; ++kt) {
            const __bf16 *ks = kring[kt % 3], *vs = vring[kt % 3];
#pragma unroll 1
            for (int s32 = 0; s32 < 2; ++s32) {
                const int kb0 = kt * BN + 32 * s32;
                if (slice_skipped(kb0)) continue;
                f32x4 bias[2];
                if (slice_masked(kb0)) make_bias(kb0, bias);
                else bias[0] = bias[1] = zero4;
                if (mode == 1) max_slice(s32, ks, bias);
                else slice(s32, ks, vs, bias);
            }
            const bool last = kt == kt_hi;
            if (last && mode == 0 && (!PREFIX || tq >= P) && tq < T) {
#pragma unroll
                for (int h = 0; h < NH; ++h) wave_restart |= !(l_part[h] <= RESTART_PART_SUM);
            }
            const int nt = !last ? kt + 1 : (mode == 1 ? kt_lo : next_lo);
            const int limit = min(min(kt, nt) + 2, mode == 1 ? kt_hi : run_last_tile);
            while (next_copy <= limit) issue_tile(next_copy++);
            if (last && mode == 0 && __any(wave_restart) && lane == 0) restart_flag[n_done & 1] = 1;
            if (next_copy - 1 > nt) wait_all_but_newest();
            else __builtin_amdgcn_s_waitcnt(0x0070);                      // vmcnt(0) lgkmcnt(0)
            bare_barrier();
        }
        return mode == 0 && __builtin_amdgcn_readfirstlane(restart_flag[n_done & 1]) != 0;
    };

    wait_vmem();
    __syncthreads();
    for (;;) {
    bool more_items = false;
    for (int qt = qt_first; qt < qt_end; ++qt) {
        t0 = q0 + qt * BM;
        tw = t0 + 16 * sub;
        tq = tw + r;
        const int kt_lo = tile_lo(qt), kt_hi = tile_hi(qt);
        const int next_lo = qt + 1 < qt_end ? tile_lo(qt + 1) : 1 << 30;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            l_part[h] = 0.f;
#pragma unroll
            for (int cb = 0; cb < D_V / 16; ++cb) o[h][cb] = zero4;
        }
        ref_pass(kt_hi);
        if (run_tiles(qt, kt_lo, kt_hi, next_lo, 0)) {
            wait_vmem();
            __syncthreads();
            if (tid == 0) restart_flag[n_done & 1] = 0;
#pragma unroll
            for (int h = 0; h < NH; ++h) m_ref[h] = -INFINITY;
            start_ring(qt);
            wait_vmem();
            __syncthreads();
            run_tiles(qt, kt_lo, kt_hi, next_lo, 1);
#pragma unroll
            for (int h = 0; h < NH; ++h) {
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

        // ---- epilogue.  Requested in this order: the first K/V tiles of what
        // comes next, this tile's gate and lambda for the wave's two signal
        // heads, the next query tile's queries; then the math and the stores.
        const bool row_ok = (!PREFIX || tq >= P) && tq < T;
        const long row = qseq0 + (row_ok ? (PREFIX ? tq - P : tq) : 0);
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
        const int e_lo = PREFIX ? max(t0, P) : t0, e_hi = min(t0 + BM, T);
        const long e_r0 = qseq0 + (PREFIX ? e_lo - P : e_lo);
        const uint32_t e_rows = (uint32_t)max(0, e_hi - e_lo);
        const auto g_rs = make_rsrc(p.gate + (e_r0 * n_sig + GROUP * j) * D_V, e_rows * (uint32_t)(n_sig * D_V * 2));
        const auto o_rs = make_rsrc(p.out + (e_r0 * n_sig + GROUP * j) * D_V, e_rows * (uint32_t)(n_sig * D_V * 2));
        const auto l_rs = make_rsrc(p.lam + e_r0 * n_sig + GROUP * j, e_rows * (uint32_t)(n_sig * 2));
        const int eln = lane_now();
        const int edt = tw + (eln & 15) - e_lo;
        const uint32_t e_off = (uint32_t)edt * (uint32_t)(n_sig * D_V * 2) + 16 * (eln >> 4);
        u32x4 gw[R::NOUT][D_V / 32];
#pragma unroll
        for (int c = 0; c < D_V / 32; ++c)
#pragma unroll
            for (int i = 0; i < R::NOUT; ++i) gw[i][c] = bld16(g_rs, e_off + R::out_head(i) * D_V * 2 + 64 * c);
        // lambda of the wave's two signal heads (adjacent: one 4-byte word)
        const uint32_t lw = __builtin_amdgcn_raw_buffer_load_b32(
            l_rs, (uint32_t)edt * (uint32_t)(n_sig * 2) + 2 * R::out_head(0), 0, 0);
        load_q(n_qt, (long)n_b * Tq, n_j);
        // output stores cover whole 128-byte lines: store k of a half writes
        // rows 8k .. 8k+7, eight 16-byte chunks each; lanes r and r ^ 8 swap the
        // chunk the other one stores (see below)
        const int ehalf = (eln & 15) >> 3;
        uint32_t so = (uint32_t)(tw + (eln & 7) - e_lo) * (uint32_t)(n_sig * D_V * 2) + 16 * (eln >> 4) + 64 * ehalf;
        asm volatile("" : "+v"(so));

        float inv[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) inv[h] = 1.f / group4_sum(l_part[h]);
        const float lam[2] = {bf16_lo(lw), bf16_hi(lw)};
        float *xch = xch_base + (sub * 64 + lane) * XCH_FLOATS;
        // two halves of 64 columns: c = 2*half, 2*half + 1
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float hn[2][8];
            if constexpr (ROLE == 0) {
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int e = 0; e < 8; ++e) hn[cc][e] = o[2][2 * (2 * half + cc) + e / 4][e % 4] * inv[2];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    *reinterpret_cast<f32x4 *>(xch + 8 * cc) = f32x4{hn[cc][0], hn[cc][1], hn[cc][2], hn[cc][3]};
                    *reinterpret_cast<f32x4 *>(xch + 8 * cc + 4) = f32x4{hn[cc][4], hn[cc][5], hn[cc][6], hn[cc][7]};
                }
            }
            if (half == 0) {
                // every K/V copy issued before this epilogue has landed (they
                // are older than its gate, lambda and query loads), so after the
                // barrier below the next query tile may read any tile in the ring
                constexpr int vm = D_V / 32 * R::NOUT + 1 + NH * KK;
                static_assert(vm < 64, "vmcnt range");
                __builtin_amdgcn_s_waitcnt((vm & 15) | ((vm >> 4) << 14) | 0x0F70);
            }
            lds_barrier();         // the half of H_N is in LDS
            if constexpr (ROLE == 1) {
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(xch + 8 * cc);
                    const f32x4 bq = *reinterpret_cast<const f32x4 *>(xch + 8 * cc + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hn[cc][e] = a[e];
                        hn[cc][4 + e] = bq[e];
                    }
                }
            }
            u32x4 yw[R::NOUT][2];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int c = 2 * half + cc;
                const int col = 32 * c + 8 * g;
#pragma unroll
                for (int i = 0; i < R::NOUT; ++i) {
                    const int h = i;   // local index of the output head
                    float y[8], hs[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t gword = gw[i][c][e / 2];
                        const float gv = (e & 1) ? bf16_hi(gword) : bf16_lo(gword);
                        hs[e] = o[h][2 * c + e / 4][e % 4] * inv[h];
                        y[e] = gv * fmaf(-lam[i], hn[cc][e], hs[e]);
                    }
                    yw[i][cc] = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                      pack_bf16x2(y[6], y[7])};
                    if constexpr (TRAIN) if (row_ok)
                        *reinterpret_cast<u32x4 *>(p.hs + (row * n_sig + GROUP * j + R::out_head(i)) * D_V + col) =
                            u32x4{pack_bf16x2(hs[0], hs[1]), pack_bf16x2(hs[2], hs[3]), pack_bf16x2(hs[4], hs[5]),
                                  pack_bf16x2(hs[6], hs[7])};
                }
                if constexpr (TRAIN && ROLE == 0) if (row_ok)
                    *reinterpret_cast<u32x4 *>(p.hn + (row * n_kv + j) * D_V + col) =
                        u32x4{pack_bf16x2(hn[cc][0], hn[cc][1]), pack_bf16x2(hn[cc][2], hn[cc][3]),
                              pack_bf16x2(hn[cc][4], hn[cc][5]), pack_bf16x2(hn[cc][6], hn[cc][7])};
            }
            // Lane r (< 8) holds chunks c0 = 2*half and c0 + 1 of row r, lane r + 8
            // those of row r + 8: the first store writes rows 0..7 (lane r: its
            // c0 chunk, lane r + 8: lane r's c0 + 1 chunk), the second rows 8..15
            // (lane r: lane r + 8's c0 chunk, lane r + 8: its own c0 + 1 chunk).
            // Each lane hands over the chunk the other one stores (16-lane row
            // rotation by 8: lane l <-> l ^ 8).
#pragma unroll
            for (int i = 0; i < R::NOUT; ++i) {
                u32x4 give, got, first, second;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    give[w] = ehalf ? yw[i][0][w] : yw[i][1][w];
                    got[w] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give[w], 0x128, 0xF, 0xF, false);
                    first[w] = ehalf ? got[w] : yw[i][0][w];
                    second[w] = ehalf ? yw[i][1][w] : got[w];
                }
                const uint32_t ho = so + R::out_head(i) * D_V * 2 + 128 * half;
                bst16(o_rs, ho, first);
                bst16(o_rs, ho + 8 * (uint32_t)(n_sig * D_V * 2), second);
            }
            if (half == 0) lds_barrier();   // B has read the first half before A overwrites it
        }
        if constexpr (TRAIN) if (row_ok && g == 0) {
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const float m = m_ref[h] == -INFINITY ? 0.f : m_ref[h];
                const int gh = R::head(h);
                const int colh = gh < GROUP ? GROUP * j + gh : n_sig + j;
                p.lse[row * (n_sig + n_kv) + colh] = m - __log2f(inv[h]);
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
    // the next item's first tiles and queries have landed in every wave; a
    // wave's last 8 memory operations are its output stores, which need not
    // complete first: vmcnt(8)
    static_assert(2 * D_V / 32 == 8, "output stores per wave");
    if constexpr (TRAIN) wait_vmem();
    else __builtin_amdgcn_s_waitcnt(0x0F78);
    bare_barrier();
    }
}

template <bool PREFIX, bool TRAIN, bool ASMC>
__global__ __launch_bounds__(THREADS, 1) void prefill_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) KRing kring;
    __shared__ __attribute__((aligned(16))) VRing vring;
    __shared__ __attribute__((aligned(16))) float xch[4 * 64 * XCH_FLOATS];
    __shared__ int restart_flag[2];
    if (__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) < 4) run<PREFIX, TRAIN, ASMC, 0>(p, kring, vring, xch, restart_flag);
    else run<PREFIX, TRAIN, ASMC, 1>(p, kring, vring, xch, restart_flag);
}

}  // namespace pf

static int compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Test knobs, read at every launch: GDLA_PREFILL_GRID caps the number of
// persistent workgroups, GDLA_PREFILL_RUN_LEN sets the query tiles per work
// item of a sliding window of up to 2*BN+1 keys.  The output does not depend
// on either (a query tile's arithmetic is the same in any schedule); the tests
// compare schedules bit for bit.
static long env_knob(const char *name) {
    const char *e = std::getenv(name);
    if (!e || !*e) return 0;
    char *end = nullptr;
    const long v = std::strtol(e, &end, 10);
    return (end && *end == 0 && v > 0) ? v : 0;
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
    p.n_qt = (P % pf::BM + Tq + pf::BM - 1) / pf::BM;
    // Sliding windows of up to 2*BN+1 keys touch at most three key tiles per
    // query tile, so a workgroup can walk a run of consecutive query tiles and
    // copy one new K/V tile per query tile; runs are sized for about two per CU.
    const int n_cu = compute_units();
    p.run_len = 1;
    if (p.window > 0 && p.window <= 2 * pf::BN + 1) {
        const long tiles = (long)B * n_kv * p.n_qt;
        p.run_len = (int)std::max(1L, std::min((long)p.n_qt, (tiles + 2L * n_cu - 1) / (2L * n_cu)));
        if (const long rl = env_knob("GDLA_PREFILL_RUN_LEN")) p.run_len = (int)std::min((long)p.n_qt, rl);
    }
    p.n_runs = (p.n_qt + p.run_len - 1) / p.run_len;
    // one persistent workgroup per CU (at most one fits: LDS and registers)
    const long items = (long)B * n_kv * p.n_runs;
    long blocks = std::min(items, (long)n_cu);
    if (const long g = env_knob("GDLA_PREFILL_GRID")) blocks = std::min(blocks, g);
    const bool runs = p.window > 0 && p.window <= 2 * pf::BN + 1;
    const dim3 grid((unsigned)blocks), block(pf::THREADS);
    if (save_hs)        // the saving mode (a full prefill only)
        hipLaunchKernelGGL((pf::prefill_kernel<false, true, false>), grid, block, 0, stream, p);
    else if (P > 0 && runs)
        hipLaunchKernelGGL((pf::prefill_kernel<true, false, true>), grid, block, 0, stream, p);
    else if (P > 0)
        hipLaunchKernelGGL((pf::prefill_kernel<true, false, false>), grid, block, 0, stream, p);
    else if (runs)
        hipLaunchKernelGGL((pf::prefill_kernel<false, false, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((pf::prefill_kernel<false, false, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

long prefill_grid_blocks(int B, int Tq, int P, int n_kv) {
    return (long)B * n_kv * ((P % pf::BM + (long)Tq + pf::BM - 1) / pf::BM);
}

}  // namespace gdla
