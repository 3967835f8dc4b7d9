// decode_gfx950.hip -- GDLA attention core for one new token per sequence.
//
// Decode reads the whole visible KV cache of every (sequence, KV head) once
// and does little arithmetic per byte, so it is bound by HBM bandwidth; the
// KV cache is what grows with the context (the report's motivation for the
// latent KV path: aitrends.kr GDLA paragraph; metalmedia P4 summary).  The
// five query heads of a group (4 signal + 1 noise) share each K/V byte read.
//
// Split-KV: workgroup (split s, KV head j, sequence b) covers one contiguous
// chunk of the visible keys; its 4 waves take 32-key blocks of the chunk in
// turn.  Per block:
//   K (A operand) is loaded straight from HBM into registers;
//   S^T = K Q^T on the matrix cores, the 5 real queries in 16 MFMA columns;
//   online softmax in base 2, as in prefill;
//   V is staged through a wave-private LDS slice, transposed, for O^T += V^T P^T.
// The 4 waves then merge (log-sum-exp) in LDS.  When a single workgroup
// covers the whole visible range -- always for a 128-key sliding window --
// it applies the combine and gate itself; otherwise it writes (m, l, acc)
// partials and a second kernel merges the splits and applies the epilogue
//   D = H_S - lambda * Repeat_4(H_N),  out = gate * D.
#include "gdla_device.h"
#include "gdla_launch.h"

#include <algorithm>

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
    float A[HEADS], Ls[HEADS];
#pragma unroll
    for (int h = 0; h < HEADS; ++h) {
        float m = -INFINITY;
        for (int s = 0; s < p.n_split; ++s) m = fmaxf(m, base[s * PART_FLOATS + h]);
        float l = 0.f, acc = 0.f;
        for (int s = 0; s < p.n_split; ++s) {
            const float *part = base + s * PART_FLOATS;
            const float f = part[h] == -INFINITY ? 0.f : fast_exp2(part[h] - m);
            l += f * part[8 + h];
            acc += f * part[16 + h * D_V + c];
        }
        Ls[h] = l;
        A[h] = acc;
    }
    decode_epilogue(p, b, j, c, load_gate_col(p, b, j, c), A, Ls);
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
    hipLaunchKernelGGL(decode_split_kernel, dim3(n_split, n_kv, B), dim3(DC_THREADS), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_split == 1) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(n_kv, B), dim3(D_V), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdla
