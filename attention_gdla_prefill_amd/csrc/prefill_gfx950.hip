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
//   2. K and V tiles stream HBM -> registers -> LDS, double buffered, shared
//      by the 4 waves and all 5 heads; V is stored transposed so that the P*V
//      contraction reads 16 contiguous bytes per lane;
//   3. S^T = K Q^T on the matrix cores (bf16 in, fp32 out), causal / window
//      mask on the tiles that straddle the band edge only;
//   4. online softmax in base 2 with the scale folded in and row sums kept
//      per lane.  Each row's reference maximum is fixed by the first visible
//      keys it meets; later keys may exceed it by up to 2^64 before the
//      workgroup restarts its pass with a raised reference (rare: it needs a
//      logit jump of ~44 in natural units).  The accumulators are thus never
//      rescaled inside the loop, which keeps them in the matrix-core register
//      file;
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

namespace gdla {

constexpr int PF_BM = 64;             // query tokens per workgroup
constexpr int PF_BN = 64;             // keys per LDS tile
constexpr int PF_THREADS = 256;       // 4 waves
constexpr int KS_ROW = D_QK + 8;      // bf16 per K row in LDS (16-byte pad against bank conflicts)
constexpr int VT_ROW = PF_BN + 8;     // bf16 per transposed V row in LDS
constexpr int KK_STEPS = D_QK / 32;   // MFMA k-steps over the query-key dim

struct PrefillParams {
    const __bf16 *qs, *qn, *k, *v, *lam, *gate;
    __bf16 *out;
    int B, T, n_kv, window;
    float scale_log2;                 // softmax scale * log2(e)
    int n_qt;                         // query tiles per sequence
};

// Workgroup index -> (head instance b*n_kv+j, query tile).  Consecutive
// workgroups go to the 8 XCDs in turn; each XCD gets a fixed subset of head
// instances so that the K/V of a head stay in one XCD's L2.  Full causal
// layers hand out the heaviest (last) query tiles first.
__device__ __forceinline__ void map_item(int bid, int n_hi, int n_qt, bool causal, int &hi, int &qt) {
    int rank;
    if ((n_hi & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3, per_xcd = n_hi >> 3;
        rank = slot / per_xcd;
        hi = (slot % per_xcd) * 8 + xcd;
    } else {
        hi = bid % n_hi;
        rank = bid / n_hi;
    }
    qt = causal ? n_qt - 1 - rank : rank;
}

__global__ __launch_bounds__(PF_THREADS, 1) void prefill_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][PF_BN * KS_ROW];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[2][D_V * VT_ROW];

    const int T = p.T, n_kv = p.n_kv, window = p.window;
    const int n_sig = n_kv * GROUP;
    int hi, qt;
    map_item(blockIdx.x, p.B * n_kv, p.n_qt, window == 0, hi, qt);
    const int b = hi / n_kv, j = hi % n_kv;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int t0 = qt * PF_BM;
    const int tw = t0 + 16 * wave;    // first query token of this wave
    const int tq = tw + r;            // query token of this lane
    const long seq0 = (long)b * T;    // first row of sequence b

    // ---- queries: B operand fragments, lane holds Q[tq][32kk + 8g .. +7]
    bf16x8 qf[HEADS][KK_STEPS];
    {
        const bool ok = tq < T;
        const __bf16 *qsrow = p.qs + ((seq0 + (ok ? tq : 0)) * n_sig + GROUP * j) * D_QK + 8 * g;
        const __bf16 *qnrow = p.qn + ((seq0 + (ok ? tq : 0)) * n_kv + j) * D_QK + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KK_STEPS; ++kk) {
#pragma unroll
            for (int h = 0; h < GROUP; ++h) {
                u32x4 w = ok ? ldg16(qsrow + h * D_QK + 32 * kk) : u32x4{0, 0, 0, 0};
                qf[h][kk] = __builtin_bit_cast(bf16x8, w);
            }
            u32x4 w = ok ? ldg16(qnrow + 32 * kk) : u32x4{0, 0, 0, 0};
            qf[GROUP][kk] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // ---- key tiles this query tile can see
    const int key_last = min(t0 + PF_BM, T) - 1;
    const int key_first = window > 0 ? max(0, t0 - window + 1) : 0;
    const int kt_lo = key_first / PF_BN, kt_hi = key_last / PF_BN;

    // ---- tile staging: K as 6 16-byte chunks per thread, V as a 4-key x 8-column block
    u32x4 kreg[6], vreg[4];
    const int v_kg = tid >> 4, v_cc = tid & 15;
    auto load_tile = [&](int kt) {
        const int kbase = kt * PF_BN;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int c = tid + PF_THREADS * i;
            const int key = kbase + c / 24, dc = c % 24;
            kreg[i] = key < T ? ldg16(p.k + ((seq0 + key) * n_kv + j) * D_QK + 8 * dc)
                              : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int key = kbase + 4 * v_kg + rr;
            vreg[rr] = key < T ? ldg16(p.v + ((seq0 + key) * n_kv + j) * D_V + 8 * v_cc)
                               : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int c = tid + PF_THREADS * i;
            *reinterpret_cast<u32x4 *>(&Ks[buf][(c / 24) * KS_ROW + 8 * (c % 24)]) = kreg[i];
        }
        u32x2 cols[8];
        transpose4x8(vreg, cols);
        const int kl0 = 4 * v_kg;
        const int pos = 32 * (kl0 >> 5) + vt_pos(kl0 & 31);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *reinterpret_cast<u32x2 *>(&Vt[buf][(8 * v_cc + e) * VT_ROW + pos]) = cols[e];
    };

    // ---- softmax state (per lane: query tq of each head)
    float m_ref[HEADS], l_part[HEADS];
    f32x4 o[HEADS][D_V / 16];
#pragma unroll
    for (int h = 0; h < HEADS; ++h) {
        m_ref[h] = -INFINITY;
        l_part[h] = 0.f;
#pragma unroll
        for (int cb = 0; cb < D_V / 16; ++cb) o[h][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float c_log2 = p.scale_log2;
    __shared__ int restart_flag;
    if (tid == 0) restart_flag = 0;
    bool wave_restart = false;        // this wave met a key beyond its reference + RESTART_LOG2

    load_tile(kt_lo);
    store_tile(0);
    __syncthreads();

    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
        const int buf = (kt - kt_lo) & 1;
        const bool more = kt < kt_hi;

#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int kb0 = kt * PF_BN + 32 * sub;     // first key of this 32-key slice
            // wave-uniform skips: no valid query, all keys in the future, all keys too old
            if (wave_restart || tw >= T || kb0 > tw + 15) continue;
            if (window > 0 && kb0 + 31 < tw - window + 1) continue;
            const bool need_mask = (kb0 + 31 > tw) || (window > 0 && kb0 < tw + 16 - window);

            // S^T = K Q^T over 2 blocks of 16 keys
            f32x4 s[HEADS][2];
#pragma unroll
            for (int h = 0; h < HEADS; ++h) s[h][0] = s[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK_STEPS; ++kk) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        &Ks[buf][(32 * sub + 16 * kb + r) * KS_ROW + 32 * kk + 8 * g]);
#pragma unroll
                    for (int h = 0; h < HEADS; ++h) s[h][kb] = mfma16(a, qf[h][kk], s[h][kb]);
                }
            }
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = kb0 + 16 * kb + 4 * g + e;
                        const bool vis = key <= tq && (window == 0 || key > tq - window);
                        if (!vis) {
#pragma unroll
                            for (int h = 0; h < HEADS; ++h) s[h][kb][e] = -INFINITY;
                        }
                    }
            }

            // reference maxima: set on first sight, restart on a jump beyond RESTART_LOG2
            bool jump = false;
#pragma unroll
            for (int h = 0; h < HEADS; ++h) {
                float mx = fmaxf(fmaxf(fmaxf(s[h][0][0], s[h][0][1]), fmaxf(s[h][0][2], s[h][0][3])),
                                 fmaxf(fmaxf(s[h][1][0], s[h][1][1]), fmaxf(s[h][1][2], s[h][1][3])));
                mx = group4_max(mx) * c_log2;
                if (m_ref[h] == -INFINITY) {
                    m_ref[h] = mx;
                } else if (mx > m_ref[h] + RESTART_LOG2) {
                    m_ref[h] = mx + RESTART_HEADROOM_LOG2;
                    jump = true;
                }
            }
            if (__any(jump)) {
                wave_restart = true;
                continue;
            }

            bf16x8 pb[HEADS];
#pragma unroll
            for (int h = 0; h < HEADS; ++h) {
                const float mref = m_ref[h] == -INFINITY ? 0.f : m_ref[h];
                float pv[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pv[e] = fast_exp2(fmaf(s[h][0][e], c_log2, -mref));
                    pv[4 + e] = fast_exp2(fmaf(s[h][1][e], c_log2, -mref));
                }
                l_part[h] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
                u32x4 w = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
                pb[h] = __builtin_bit_cast(bf16x8, w);
            }

            // O^T += V^T P^T
#pragma unroll
            for (int cb = 0; cb < D_V / 16; ++cb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                    &Vt[buf][(16 * cb + r) * VT_ROW + 32 * sub + 8 * g]);
#pragma unroll
                for (int h = 0; h < HEADS; ++h) o[h][cb] = mfma16(a, pb[h], o[h][cb]);
            }
        }

        if (more) {
            load_tile(kt + 1);
            store_tile(buf ^ 1);
        }
        if (wave_restart && lane == 0) restart_flag = 1;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(restart_flag)) {
            // some row met a key far above its reference: redo the pass from the
            // first tile with the raised references (accumulators start from zero)
            __syncthreads();                       // every wave has read the flag
            if (tid == 0) restart_flag = 0;
#pragma unroll
            for (int h = 0; h < HEADS; ++h) {
                l_part[h] = 0.f;
#pragma unroll
                for (int cb = 0; cb < D_V / 16; ++cb) o[h][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            wave_restart = false;
            load_tile(kt_lo);
            store_tile(0);
            __syncthreads();
            kt = kt_lo - 1;
        }
    }

    // ---- epilogue: normalise, differential combine, gate, bf16 store
    float inv[HEADS];
#pragma unroll
    for (int h = 0; h < HEADS; ++h) inv[h] = 1.f / group4_sum(l_part[h]);
    if (tq >= T) return;

    const long row = seq0 + tq;
    const u32x2 lw = *reinterpret_cast<const u32x2 *>(p.lam + row * n_sig + GROUP * j);
    const float lam[GROUP] = {bf16_lo(lw[0]), bf16_hi(lw[0]), bf16_lo(lw[1]), bf16_hi(lw[1])};
#pragma unroll
    for (int cb = 0; cb < D_V / 16; ++cb) {
        const int c = 16 * cb + 4 * g;
        float hn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hn[e] = o[GROUP][cb][e] * inv[GROUP];
#pragma unroll
        for (int h = 0; h < GROUP; ++h) {
            const long off = (row * n_sig + GROUP * j + h) * D_V + c;
            const u32x2 gw = *reinterpret_cast<const u32x2 *>(p.gate + off);
            const float gv[4] = {bf16_lo(gw[0]), bf16_hi(gw[0]), bf16_lo(gw[1]), bf16_hi(gw[1])};
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // H_S and H_N are formed the same way, so identical queries with
                // lambda = 1 give exactly 0
                const float hs = o[h][cb][e] * inv[h];
                y[e] = gv[e] * fmaf(-lam[h], hn[e], hs);
            }
            *reinterpret_cast<u32x2 *>(p.out + off) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
    }
}

hipError_t launch_prefill(const void *qs, const void *qn, const void *k, const void *v,
                          const void *lam, const void *gate, void *out, int B, int T, int n_kv,
                          int window, float scale, hipStream_t stream) {
    PrefillParams p;
    p.qs = static_cast<const __bf16 *>(qs);
    p.qn = static_cast<const __bf16 *>(qn);
    p.k = static_cast<const __bf16 *>(k);
    p.v = static_cast<const __bf16 *>(v);
    p.lam = static_cast<const __bf16 *>(lam);
    p.gate = static_cast<const __bf16 *>(gate);
    p.out = static_cast<__bf16 *>(out);
    p.B = B;
    p.T = T;
    p.n_kv = n_kv;
    p.window = window >= T ? 0 : window;     // a window covering the sequence is full causal
    p.scale_log2 = scale * LOG2E;
    p.n_qt = (T + PF_BM - 1) / PF_BM;
    const long blocks = (long)B * n_kv * p.n_qt;
    hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)blocks), dim3(PF_THREADS), 0, stream, p);
    return hipGetLastError();
}

long prefill_grid_blocks(int B, int T, int n_kv) {
    return (long)B * n_kv * ((T + PF_BM - 1) / PF_BM);
}

}  // namespace gdla
