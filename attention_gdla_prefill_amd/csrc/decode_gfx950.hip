// decode_gfx950.hip -- GDLA attention core for one new token per sequence.
//
// Decode reads the whole visible KV cache of every (sequence, KV head) once
// and does little arithmetic per byte, so it is bound by HBM bandwidth; the
// KV cache is what grows with the context (idailynews, "연속기획⑩ 독자 AI 2차
// 평가 Motif 3 모델과 인프라 함께 설계", section "GDLA로 긴 문맥과 메모리 부담
// 함께 다뤄": the cache grows with the context and the sliding-window layers
// cover 128 tokens; aitrends.kr, GDLA paragraph: the latent KV path exists to
// shrink it).  The five query heads of a group (4 signal + 1 noise) share
// each K/V byte read.
//
// Split-KV: workgroup (split s, KV head j, sequence b) covers one contiguous
// chunk of the visible keys; its 4 waves take 32-key blocks of the chunk in
// turn.  Per block:
//   K (A operand) is loaded straight from HBM into registers;
//   S^T = K Q^T on the matrix cores, the 5 real queries in 16 MFMA columns;
//   online softmax in base 2, as in prefill;
//   V is staged through a wave-private LDS slice, transposed, for O^T += V^T P^T.
// The 4 waves then merge (log-sum-exp) in LDS.  When a single workgroup
// covers the whole visible range it applies the combine and gate itself;
// otherwise it writes (m, l, acc) partials and a second kernel merges the
// splits and applies the epilogue
//   D = H_S - lambda * Repeat_4(H_N),  out = gate * D.
// A sliding window of up to 128 keys takes its own kernel (decode_window_kernel,
// below): one workgroup per (sequence, KV head) that requests all of its loads
// at once.
#include "gdla_device.h"
#include "gdla_launch.h"

#include <algorithm>
#include <mutex>

namespace gdla {

constexpr int DC_THREADS = 256;
constexpr int DC_WAVES = 4;
constexpr int DC_BLOCK = 32;            // keys per wave step
constexpr int DC_CHUNK = 2048;          // target keys per workgroup
constexpr int DCV_ROW = DC_BLOCK + 8;   // bf16 per transposed V row in LDS
constexpr int PART_FLOATS = 16 + HEADS * D_V;   // m[8] | l[8] | acc[5][128]

struct DecodeParams {
    const __bf16 *qs, *qn, *kc, *vc, *lam, *gate;
    const int32_t *cu;
    __bf16 *out;
    float *ws;
    int n_kv, n_split, window;
    float scale_log2;
};

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// gate and lambda of column c of the 4 signal heads of group (b, j)
struct GateCol {
    __bf16 gate[GROUP], lam[GROUP];
};

__device__ __forceinline__ GateCol load_gate_col(const DecodeParams &p, int b, int j, int c) {
    GateCol gc;
    const int n_sig = p.n_kv * GROUP;
#pragma unroll
    for (int h = 0; h < GROUP; ++h) {
        const long hrow = (long)b * n_sig + GROUP * j + h;
        gc.lam[h] = p.lam[hrow];
        gc.gate[h] = p.gate[hrow * D_V + c];
    }
    return gc;
}

// out[b, 4j+h, c] = gate * (A_h / L_h - lambda_h * A_n / L_n) for h = 0..3
__device__ __forceinline__ void decode_epilogue(const DecodeParams &p, int b, int j, int c,
                                                const GateCol &gc, const float A[HEADS],
                                                const float L[HEADS]) {
    const int n_sig = p.n_kv * GROUP;
    const float hn = L[GROUP] > 0.f ? A[GROUP] / L[GROUP] : 0.f;
#pragma unroll
    for (int h = 0; h < GROUP; ++h) {
        const long hrow = (long)b * n_sig + GROUP * j + h;
        const float hs = L[h] > 0.f ? A[h] / L[h] : 0.f;
        p.out[hrow * D_V + c] = (__bf16)((float)gc.gate[h] * fmaf(-(float)gc.lam[h], hn, hs));
    }
}

__global__ __launch_bounds__(DC_THREADS) void decode_split_kernel(DecodeParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 Vt[DC_WAVES][D_V * DCV_ROW];
    __shared__ float red_m[DC_WAVES][HEADS], red_l[DC_WAVES][HEADS];
    __shared__ float red_o[DC_WAVES][HEADS][D_V];

    const int sp = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int n_kv = p.n_kv, n_sig = n_kv * GROUP;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;

    // with one split the epilogue runs here: its gate and lambda load first
    GateCol gc{};
    if (p.n_split == 1 && tid < D_V) gc = load_gate_col(p, b, j, tid);
    const int start = p.cu[b];
    const int L = p.cu[b + 1] - start;
    const int vis_lo = p.window > 0 ? max(0, L - p.window) : 0;
    const int n_vis = max(0, L - vis_lo);
    int chunk = (n_vis + p.n_split - 1) / p.n_split;
    chunk = (chunk + DC_BLOCK - 1) & ~(DC_BLOCK - 1);
    const int k_begin = vis_lo + sp * chunk;          // relative to the sequence start
    const int k_end = min(L, k_begin + chunk);

    // queries: column r of the B operand; r < 4 signal head 4j+r, r == 4 noise head j
    bf16x8 qf[D_QK / 32];
    {
        const __bf16 *src = r < GROUP ? p.qs + ((long)b * n_sig + GROUP * j + r) * D_QK
                                      : p.qn + ((long)b * n_kv + j) * D_QK;
#pragma unroll
        for (int kk = 0; kk < D_QK / 32; ++kk) {
            u32x4 w = r < HEADS ? ldg16(src + 32 * kk + 8 * g) : u32x4{0, 0, 0, 0};
            qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }

    float m_ref = -INFINITY, l_part = 0.f;
    f32x4 o[D_V / 16];
#pragma unroll
    for (int cb = 0; cb < D_V / 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    __bf16 *vt = Vt[wave];
    const float c_log2 = p.scale_log2;
    const __bf16 *kbase = p.kc + ((long)start * n_kv + j) * D_QK;
    const __bf16 *vbase = p.vc + ((long)start * n_kv + j) * D_V;
    const long krow = (long)n_kv * D_QK, vrow = (long)n_kv * D_V;

    for (int kb0 = k_begin + DC_BLOCK * wave; kb0 < k_end; kb0 += DC_BLOCK * DC_WAVES) {
        // K straight into A-operand fragments: lane holds K[kb0 + 16kb + r][32kk + 8g .. +7]
        bf16x8 ka[2][D_QK / 32];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // keys past the chunk read its last key (their scores are masked
            // below and their weights are 0), so the loads need no branch
            const int key = min(kb0 + 16 * kb + r, k_end - 1);
            const __bf16 *src = kbase + (long)key * krow + 8 * g;
#pragma unroll
            for (int kk = 0; kk < D_QK / 32; ++kk) ka[kb][kk] = __builtin_bit_cast(bf16x8, ldg16(src + 32 * kk));
        }
        // V block: each lane takes 2 units of 4 keys x 8 columns
        u32x4 vr[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int kg = (lane >> 4) + 4 * i, cc = lane & 15;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = min(kb0 + 4 * kg + rr, k_end - 1);
                vr[i][rr] = ldg16(vbase + (long)key * vrow + 8 * cc);
            }
        }

        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < D_QK / 32; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = mfma16(ka[kb][kk], qf[kk], s[kb]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (kb0 + 16 * kb + 4 * g + e >= k_end) s[kb][e] = -INFINITY;

        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mx = group4_max(mx) * c_log2;
        const float m_new = fmaxf(m_ref, mx);
        const bool raise = m_new > m_ref + RESCALE_LOG2;
        if (__any(raise)) {
            const float alpha = raise ? fast_exp2(m_ref - m_new) : 1.f;
            m_ref = raise ? m_new : m_ref;
            l_part *= alpha;
#pragma unroll
            for (int cb = 0; cb < D_V / 16; ++cb) o[cb] *= alpha;
        }
        const float mref = m_ref == -INFINITY ? 0.f : m_ref;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pv[e] = fast_exp2(fmaf(s[0][e], c_log2, -mref));
            pv[4 + e] = fast_exp2(fmaf(s[1][e], c_log2, -mref));
        }
        l_part += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        const u32x4 pw = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                          pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);

        wave_lds_sync();                  // the previous block's reads of vt are done
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int kg = (lane >> 4) + 4 * i, cc = lane & 15;
            u32x2 cols[8];
            transpose4x8(vr[i], cols);
            const int pos = vt_pos(4 * kg);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<u32x2 *>(&vt[(8 * cc + e) * DCV_ROW + pos]) = cols[e];
        }
        wave_lds_sync();
#pragma unroll
        for (int cb = 0; cb < D_V / 16; ++cb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&vt[(16 * cb + r) * DCV_ROW + 8 * g]);
            o[cb] = mfma16(a, pb, o[cb]);
        }
    }

    // merge the 4 waves (log-sum-exp) through LDS
    const float l_tot = group4_sum(l_part);
    if (r < HEADS) {
        if (g == 0) {
            red_m[wave][r] = m_ref;
            red_l[wave][r] = l_tot;
        }
#pragma unroll
        for (int cb = 0; cb < D_V / 16; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) red_o[wave][r][16 * cb + 4 * g + e] = o[cb][e];
    }
    __syncthreads();
    if (tid >= D_V) return;
    const int c = tid;
    float M[HEADS], Ls[HEADS], A[HEADS];
#pragma unroll
    for (int h = 0; h < HEADS; ++h) {
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < DC_WAVES; ++w) m = fmaxf(m, red_m[w][h]);
        float l = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < DC_WAVES; ++w) {
            const float f = red_m[w][h] == -INFINITY ? 0.f : fast_exp2(red_m[w][h] - m);
            l += f * red_l[w][h];
            acc += f * red_o[w][h][c];
        }
        M[h] = m;
        Ls[h] = l;
        A[h] = acc;
    }
    if (p.n_split == 1) {
        decode_epilogue(p, b, j, c, gc, A, Ls);
        return;
    }
    float *part = p.ws + (((long)b * n_kv + j) * p.n_split + sp) * PART_FLOATS;
    if (c < HEADS) {
        part[c] = M[c];
        part[8 + c] = Ls[c];
    }
#pragma unroll
    for (int h = 0; h < HEADS; ++h) part[16 + h * D_V + c] = A[h];
}

__global__ __launch_bounds__(D_V) void decode_combine_kernel(DecodeParams p) {
    const int j = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
    const float *base = p.ws + ((long)b * p.n_kv + j) * p.n_split * PART_FLOATS;
    const int ns = p.n_split;
    // the splits' maxima of the 5 heads (the same words for every thread)
    float m[HEADS];
#pragma unroll
    for (int h = 0; h < HEADS; ++h) m[h] = -INFINITY;
    for (int s = 0; s < ns; ++s)
#pragma unroll
        for (int h = 0; h < HEADS; ++h) m[h] = fmaxf(m[h], base[s * PART_FLOATS + h]);
    // then every split's sums and column c of its outputs, four splits' loads
    // in flight at a time
    float Ls[HEADS], A[HEADS];
#pragma unroll
    for (int h = 0; h < HEADS; ++h) Ls[h] = A[h] = 0.f;
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
        const float *part = base + s * PART_FLOATS;
#pragma unroll
        for (int h = 0; h < HEADS; ++h) {
            const float f = part[h] == -INFINITY ? 0.f : fast_exp2(part[h] - m[h]);
            Ls[h] += f * part[8 + h];
            A[h] += f * part[16 + h * D_V + c];
        }
    }
    decode_epilogue(p, b, j, c, load_gate_col(p, b, j, c), A, Ls);
}

// ---- window decode: every visible key of a (sequence, KV head) in one
// workgroup, no partials ------------------------------------------------------
//
// A 128-key window (the report's sliding-window layers) makes each
// (sequence, KV head) a short, independent job: 80 KB of K and V, five query
// heads.  Its time is the latency of one pass over HBM, so the kernel issues
// every load of the job at its start -- queries, K straight into matrix-core
// operand registers, V straight into LDS (direct buffer -> LDS loads), the
// gate and lambda -- and keeps LDS at 37 KB so that all (sequence, KV head)
// workgroups of a 64-sequence batch are resident at once (four per CU).
//   wave w: keys 32w .. 32w+31 of the window; S^T = K Q^T (12 MFMAs);
//   the row maxima meet in LDS (one barrier), so every wave takes its weights
//   against the same reference and nothing is rescaled;
//   O^T += V^T P^T with V^T read by the transposing LDS read;
//   the four partial sums meet in LDS (second barrier) and 64 threads apply
//   the combine and the gate, 16 bytes each.
constexpr int DW_KEYS = 128;                  // keys per workgroup: 4 waves x 32
constexpr int DW_VCH = D_V / 8 + 2;           // 16-byte chunks per padded V row in LDS (32-byte pad)
constexpr int DW_VROW = DW_VCH * 8;           // bf16 per padded V row
constexpr int DW_VROWS_PER_COPY = 3;          // a copy instruction covers 3 rows (54 of 64 lanes)
constexpr int DW_WAVE_COPIES = (32 + DW_VROWS_PER_COPY - 1) / DW_VROWS_PER_COPY;   // 11
static_assert(DW_VROWS_PER_COPY * DW_VCH <= 64, "rows per copy");
static_assert(HEADS * D_V * 4 <= 32 * DW_VROW * 2, "a wave's partial sums fit its V rows");

typedef short dw_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dw_s16x4 dw_lds_s16x4_t;
typedef __attribute__((address_space(3))) void dw_lds_void_t;

// Buffer resource over `bytes` bytes from `base`: reads at or past the size
// return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dw_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__global__ __launch_bounds__(DC_THREADS) void decode_window_kernel(DecodeParams p) {
    // V rows of the window, padded (the padding keeps the transposing reads of
    // 16 consecutive rows free of bank conflicts); after its products, wave w
    // reuses its own 32 rows for its partial sums
    __shared__ __attribute__((aligned(16))) __bf16 Vs[DW_KEYS * DW_VROW];
    __shared__ float red_m[DC_WAVES][16], red_l[DC_WAVES][16];

    const int j = blockIdx.x, b = blockIdx.y;
    const int n_kv = p.n_kv, n_sig = n_kv * GROUP;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);

    // ---- every load of the job, before any wait.  The sequence offsets are
    // read first, as a vector load: the queries, the gate and lambda (which do
    // not depend on them) follow at once, and the wait for the offsets is then
    // a count of the loads behind them, not a full drain.
    const auto cu_rs = dw_rsrc(p.cu, (gridDim.y + 1) * 4u);
    const u32x2 cuv = __builtin_amdgcn_raw_buffer_load_b64(cu_rs, 4u * b, 0, 0);   // cu[b], cu[b+1]
    // queries: column r of the B operand; r < 4 signal head 4j+r, r == 4 noise
    // head j, the other columns read zeros (an empty resource)
    bf16x8 qf[D_QK / 32];
    {
        // two resources, each uniform over the wave; a lane's offset lies past
        // the one that does not hold its query, which then reads zeros
        const auto qs_rs = dw_rsrc(p.qs + ((long)b * n_sig + GROUP * j) * D_QK, GROUP * D_QK * 2);
        const auto qn_rs = dw_rsrc(p.qn + ((long)b * n_kv + j) * D_QK, D_QK * 2);
        const uint32_t far = 1u << 30;
        const uint32_t os = r < GROUP ? (uint32_t)r * D_QK * 2 + 16 * g : far;
        const uint32_t on = r == GROUP ? 16u * g : far;
#pragma unroll
        for (int kk = 0; kk < D_QK / 32; ++kk) {
            const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(qs_rs, os + 64 * kk, 0, 0);
            const u32x4 n = __builtin_amdgcn_raw_buffer_load_b128(qn_rs, on + 64 * kk, 0, 0);
            qf[kk] = __builtin_bit_cast(bf16x8, a | n);
        }
    }
    // epilogue operands: thread t < 64 forms signal head 4j + t/16, columns
    // 8(t%16) .. +7
    // (wave 0 only: the other waves' resources are empty and read zeros, so
    // the loads carry no branch and nothing waits for them before their use)
    const int eh = (tid >> 4) & 3, ec = 8 * (tid & 15);
    const long orow0 = (long)b * n_sig + GROUP * j;                 // signal head 4j
    const auto g_rs = dw_rsrc(p.gate + orow0 * D_V, uwave == 0 ? GROUP * D_V * 2 : 0);
    const auto l_rs = dw_rsrc(p.lam + orow0, uwave == 0 ? GROUP * 2 : 0);
    const u32x4 gw = __builtin_amdgcn_raw_buffer_load_b128(g_rs, (uint32_t)(eh * D_V + ec) * 2, 0, 0);
    const u32x2 lw = __builtin_amdgcn_raw_buffer_load_b64(l_rs, 0, 0, 0);   // lambda of the 4 signal heads

    const int start = __builtin_amdgcn_readfirstlane((int)cuv[0]);
    const int L = __builtin_amdgcn_readfirstlane((int)cuv[1]) - start;
    const int vis_lo = max(0, L - p.window);
    const int n_vis = max(0, L - vis_lo);          // <= DW_KEYS
    const long row0 = (long)start + vis_lo;        // first visible cache row

    const uint32_t krow_b = (uint32_t)n_kv * D_QK * 2, vrow_b = (uint32_t)n_kv * D_V * 2;
    const auto k_rs = dw_rsrc(p.kc + (row0 * n_kv + j) * D_QK, (uint32_t)n_vis * krow_b);
    const auto v_rs = dw_rsrc(p.vc + (row0 * n_kv + j) * D_V, (uint32_t)n_vis * vrow_b);
    // V rows 32w .. 32w+31 -> LDS, three rows per instruction
    {
        const int v_lr = lane / DW_VCH, v_ch = lane % DW_VCH;
        const bool v_on = v_lr < DW_VROWS_PER_COPY && v_ch < D_V / 8;
        const uint32_t v_lane = v_lr * vrow_b + 16 * v_ch;
#pragma unroll
        for (int c = 0; c < DW_WAVE_COPIES; ++c) {
            const int rw = 32 * uwave + DW_VROWS_PER_COPY * c;        // first row of this copy
            if (v_on && DW_VROWS_PER_COPY * c + v_lr < 32)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rs, (dw_lds_void_t *)(Vs + rw * DW_VROW), 16,
                                                         v_lane + (uint32_t)rw * vrow_b, 0, 0, 0);
        }
    }
    // K rows 32w + 16kb + r as A fragments: lane holds K[..][32kk + 8g .. +7]
    bf16x8 ka[2][D_QK / 32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < D_QK / 32; ++kk)
            ka[kb][kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                k_rs, (uint32_t)(32 * uwave + 16 * kb + r) * krow_b + 64 * kk + 16 * g, 0, 0));
    // ---- scores: S^T = K Q^T, keys past the window masked by the initial value
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[kb][e] = 32 * uwave + 16 * kb + 4 * g + e < n_vis ? 0.f : -INFINITY;
#pragma unroll
        for (int kk = 0; kk < D_QK / 32; ++kk) s[kb] = mfma16(ka[kb][kk], qf[kk], s[kb]);
    }
    const float c_log2 = p.scale_log2;
    {
        const float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                               fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        const float wm = group4_max(mx);
        if (g == 0) red_m[wave][r] = wm;
    }
    __syncthreads();
    const float m = fmaxf(fmaxf(red_m[0][r], red_m[1][r]), fmaxf(red_m[2][r], red_m[3][r]));
    const float m_ref = m == -INFINITY ? 0.f : m * c_log2;
    uint32_t pw[4];
    float l_part = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = fast_exp2(fmaf(s[kb][e], c_log2, -m_ref));
        pw[2 * kb] = pack_bf16x2(pv[0], pv[1]);
        pw[2 * kb + 1] = pack_bf16x2(pv[2], pv[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) l_part = sum_bf16x2(pw[i], l_part);   // the bf16 weights P*V takes
    const float wl = group4_sum(l_part);
    if (g == 0) red_l[wave][r] = wl;
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});

    // ---- O^T += V^T P^T over this wave's 32 keys (V rows in LDS once this
    // wave's copies have landed)
    __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): this wave's copies are in LDS
    const __bf16 *vrd = Vs + (32 * uwave + 4 * g + (r >> 2)) * DW_VROW + 8 * (r & 3);
    f32x4 o[D_V / 16];
#pragma unroll
    for (int cb = 0; cb < D_V / 16; ++cb) {
        const int cc = 32 * (cb >> 1) + 4 * (cb & 1);
        const dw_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds_s16x4_t *)(vrd + cc));
        const dw_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds_s16x4_t *)(vrd + 16 * DW_VROW + cc));
        const dw_s16x4 v8[2] = {lo, hi};
        o[cb] = mfma16(__builtin_bit_cast(bf16x8, v8), pb, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    // this wave's partial sums over its own V rows (its reads are done: the
    // products above consumed them): part[h][col], lane (r, g) holds columns
    // 32c + 8g .. +7 of query r
    float *part = reinterpret_cast<float *>(Vs + 32 * uwave * DW_VROW);
    if (r < HEADS) {
#pragma unroll
        for (int c = 0; c < D_V / 32; ++c) {
            *reinterpret_cast<f32x4 *>(part + r * D_V + 32 * c + 8 * g) = o[2 * c];
            *reinterpret_cast<f32x4 *>(part + r * D_V + 32 * c + 8 * g + 4) = o[2 * c + 1];
        }
    }
    __syncthreads();
    if (tid >= 64) return;

    // ---- combine and gate: signal head 4j + eh, columns ec .. ec+7
    float ls = 0.f, ln = 0.f;
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) {
        ls += red_l[w][eh];
        ln += red_l[w][GROUP];
    }
    float hs[8] = {0, 0, 0, 0, 0, 0, 0, 0}, hn[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) {
        const float *pw_ = reinterpret_cast<const float *>(Vs + 32 * w * DW_VROW);
        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(pw_ + eh * D_V + ec);
        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(pw_ + eh * D_V + ec + 4);
        const f32x4 n0 = *reinterpret_cast<const f32x4 *>(pw_ + GROUP * D_V + ec);
        const f32x4 n1 = *reinterpret_cast<const f32x4 *>(pw_ + GROUP * D_V + ec + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hs[e] += s0[e];
            hs[4 + e] += s1[e];
            hn[e] += n0[e];
            hn[4 + e] += n1[e];
        }
    }
    const float is = ls > 0.f ? 1.f / ls : 0.f, in = ln > 0.f ? 1.f / ln : 0.f;
    const uint32_t lword = lw[eh >> 1];
    const float lam = (eh & 1) ? bf16_hi(lword) : bf16_lo(lword);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t gword = gw[e / 2];
        const float gv = (e & 1) ? bf16_hi(gword) : bf16_lo(gword);
        y[e] = gv * fmaf(-lam, hn[e] * in, hs[e] * is);
    }
    *reinterpret_cast<u32x4 *>(p.out + (orow0 + eh) * D_V + ec) =
        u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
}

int decode_splits(int max_seqlen_k, int window) {
    const long vis = window > 0 ? (long)std::min(max_seqlen_k, window) : (long)max_seqlen_k;
    const long n = (vis + DC_CHUNK - 1) / DC_CHUNK;
    return (int)std::max(1L, std::min(n, 4096L));
}

size_t decode_workspace_bytes(int B, int n_kv, int n_split) {
    return n_split > 1 ? (size_t)B * n_kv * n_split * PART_FLOATS * sizeof(float) : 0;
}

hipError_t launch_decode(const void *qs, const void *qn, const void *kc, const void *vc,
                         const int32_t *cu_seqlens, const void *lam, const void *gate, void *out,
                         void *workspace, int B, int n_kv, int n_split, int window, float scale,
                         hipStream_t stream) {
    DecodeParams p;
    p.qs = static_cast<const __bf16 *>(qs);
    p.qn = static_cast<const __bf16 *>(qn);
    p.kc = static_cast<const __bf16 *>(kc);
    p.vc = static_cast<const __bf16 *>(vc);
    p.lam = static_cast<const __bf16 *>(lam);
    p.gate = static_cast<const __bf16 *>(gate);
    p.cu = cu_seqlens;
    p.out = static_cast<__bf16 *>(out);
    p.ws = static_cast<float *>(workspace);
    p.n_kv = n_kv;
    p.n_split = n_split;
    p.window = window;
    p.scale_log2 = scale * LOG2E;
    if (window >= 1 && window <= DW_KEYS) {      // every query sees at most 128 keys: one workgroup each
        hipLaunchKernelGGL(decode_window_kernel, dim3(n_kv, B), dim3(DC_THREADS), 0, stream, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(decode_split_kernel, dim3(n_split, n_kv, B), dim3(DC_THREADS), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_split == 1) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(n_kv, B), dim3(D_V), 0, stream, p);
    return hipGetLastError();
}

// ---- scratch for callers that cannot allocate (gdla_decode_noalloc) -------
//
// The split partials of gdla_decode_noalloc live in this file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not the device array: its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and only that
// address is passed to the kernels.  Every call on one GPU shares the array,
// so calls that overlap on one GPU (different streams, no ordering) race.
// Nothing in it needs to start at zero: every split writes its whole partial
// before the combine reads it.
static __device__ __align__(256) unsigned char scratch[DECODE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void *scratch_ptr[MAX_DEVICES];
}  // namespace

hipError_t decode_noalloc_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gdla
