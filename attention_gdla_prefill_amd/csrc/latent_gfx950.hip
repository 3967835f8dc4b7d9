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
//   2. latent_split_kernel: split-KV attention of all query heads of a
//      sequence over a chunk of its latent rows -- each row read from HBM once
//      for all heads: per chunk the row maximum m, the sum l and the latent
//      output o~ = sum_s p_s c_s (512 values) per head;
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
constexpr int LT_HEADS_PER_WG = 80;       // query heads one workgroup serves (5 waves)
constexpr int LT_WAVES = LT_HEADS_PER_WG / 16;
constexpr int LT_THREADS = 64 * LT_WAVES;
constexpr int LT_BN = 32;                 // keys per LDS tile
constexpr int LT_SLOTS = 4;               // ring of tiles, copied up to 3 ahead
constexpr int LT_KK = LT_ROW / 32;        // 18 MFMA k-steps over a latent row
// LDS rows: the c part with a 32-byte pad (conflict-free 16-row fragment reads),
// the rotary part packed (8 rows per copy instruction)
constexpr int LT_CS = LT_C + 16;          // bf16 per c row in LDS (1056 bytes)
constexpr int LT_CHUNK = 4096;            // target keys per workgroup (split)

struct LatentParams {
    const __bf16 *qs, *qn, *lat, *wuk, *wuv, *lam, *gate;
    const int32_t *cu;
    __bf16 *out;
    __bf16 *qt;              // workspace: absorbed queries [B][n_q][576]
    float *part_ml;          // workspace: [B][n_split][n_q][2]  (m in log2 units, l)
    float *part_o;           // workspace: [B][n_split][n_q][512]
    int B, n_kv, n_split, window;
    float scale_log2;
};

// ---- 1. absorbed queries.  Workgroup (KV head j, 4 sequences): 512 threads,
// thread c forms q~[c] of the 5 heads of group j for the 4 sequences (20 dot
// products of 128), reading column c of W_uk[j] once.
constexpr int LT_ABS_SEQ = 4;

__global__ __launch_bounds__(LT_C) void latent_absorb_kernel(LatentParams p) {
    __shared__ float qc[LT_ABS_SEQ * HEADS][LT_KC];
    const int j = blockIdx.x, b0 = blockIdx.y * LT_ABS_SEQ, c = threadIdx.x;
    const int n_sig = p.n_kv * GROUP, n_q = n_sig + p.n_kv;
    // content parts of the 5 queries of group j for the 4 sequences
    for (int i = c; i < LT_ABS_SEQ * HEADS * LT_KC; i += LT_C) {
        const int row = i / LT_KC, d = i % LT_KC, sb = row / HEADS, h = row % HEADS;
        const int b = b0 + sb;
        float x = 0.f;
        if (b < p.B) {
            const __bf16 *q = h < GROUP ? p.qs + ((long)b * n_sig + GROUP * j + h) * D_QK
                                        : p.qn + ((long)b * p.n_kv + j) * D_QK;
            x = (float)q[d];
        }
        qc[row][d] = x;
    }
    __syncthreads();
    float acc[LT_ABS_SEQ * HEADS];
#pragma unroll
    for (int i = 0; i < LT_ABS_SEQ * HEADS; ++i) acc[i] = 0.f;
    const __bf16 *w = p.wuk + (long)j * LT_KC * LT_C + c;
    for (int d = 0; d < LT_KC; ++d) {
        const float wv = (float)w[(long)d * LT_C];
#pragma unroll
        for (int i = 0; i < LT_ABS_SEQ * HEADS; ++i) acc[i] = fmaf(qc[i][d], wv, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < LT_ABS_SEQ * HEADS; ++i) {
        const int b = b0 + i / HEADS, h = i % HEADS;
        if (b >= p.B) continue;
        const int q = h < GROUP ? GROUP * j + h : n_sig + j;
        __bf16 *dst = p.qt + ((long)b * n_q + q) * LT_ROW;
        dst[c] = (__bf16)acc[i];
        if (c < LT_R) {            // the rotary part is copied unchanged
            const __bf16 *src = h < GROUP ? p.qs + ((long)b * n_sig + GROUP * j + h) * D_QK
                                          : p.qn + ((long)b * p.n_kv + j) * D_QK;
            dst[LT_C + c] = src[LT_KC + c];
        }
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
__device__ __forceinline__ void lt_copy16(const lt_i32x4 &rsrc, uint32_t byte_off, const __bf16 *lds) {
    const uint32_t a = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) __bf16 *)lds);
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(byte_off), "s"(rsrc), "{m0}"(a) : "memory");
}

__device__ __forceinline__ lt_s16x4 lt_read_tr16(const __bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lt_lds_s16x4_t *)(p));
}

// ---- 2. split-KV attention over latent rows.  Workgroup (split, sequence,
// group of 80 query heads); wave w serves query heads 16w .. 16w+15 (the MFMA
// N dimension), all waves walk every key of the chunk.
__global__ __launch_bounds__(LT_THREADS, 1) void latent_split_kernel(LatentParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 Cring[LT_SLOTS][LT_BN * LT_CS];
    __shared__ __attribute__((aligned(16))) __bf16 Rring[LT_SLOTS][LT_BN * LT_R];

    const int sp = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
    const int n_sig = p.n_kv * GROUP, n_q = n_sig + p.n_kv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int q_row = hg * LT_HEADS_PER_WG + 16 * wave + r;      // this lane's query head
    const bool q_ok = q_row < n_q;

    const int start = p.cu[b];
    const int L = p.cu[b + 1] - start;
    const int vis_lo = p.window > 0 ? max(0, L - p.window) : 0;
    const int n_vis = max(0, L - vis_lo);
    const int chunk = (n_vis + p.n_split - 1) / p.n_split;
    const int k_begin = vis_lo + sp * chunk;                       // relative to the sequence start
    const int k_end = min(L, k_begin + chunk);
    const int n_tiles = k_end > k_begin ? (k_end - k_begin + LT_BN - 1) / LT_BN : 0;

    // absorbed query of this lane's head: B operand, lane holds q~[32kk + 8g .. +7]
    bf16x8 qf[LT_KK];
    {
        const __bf16 *src = p.qt + ((long)b * n_q + (q_ok ? q_row : 0)) * LT_ROW + 8 * g;
#pragma unroll
        for (int kk = 0; kk < LT_KK; ++kk) {
            u32x4 w = q_ok ? ldg16(src + 32 * kk) : u32x4{0, 0, 0, 0};
            qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // copies: rows of this sequence from k_begin on; rows past the sequence end read as zeros
    const __bf16 *row0 = p.lat + ((long)start + k_begin) * LT_ROW;
    const uint32_t bytes = (uint32_t)max(0, L - k_begin) * (LT_ROW * 2);
    const uint64_t row0a = reinterpret_cast<uint64_t>(row0);
    const lt_i32x4 rsrc = {(int)(uint32_t)row0a, (int)(uint32_t)(row0a >> 32), (int)bytes, 0x00020000};
    // one instruction copies one row's c part (64 lanes x 16 bytes) or the
    // rotary parts of 8 rows (lane -> row lane/8, 16-byte chunk lane%8)
    auto issue_tile = [&](int t) {
        __bf16 *cs = Cring[t % LT_SLOTS], *rs = Rring[t % LT_SLOTS];
        const uint32_t tb = (uint32_t)t * LT_BN * (LT_ROW * 2);
        for (int i = wave; i < LT_BN + LT_BN / 8; i += LT_WAVES) {
            if (i < LT_BN) {
                lt_copy16(rsrc, tb + i * (LT_ROW * 2) + 16 * lane, cs + i * LT_CS);
            } else {
                const int r8 = 8 * (i - LT_BN);
                lt_copy16(rsrc, tb + (r8 + lane / 8) * (LT_ROW * 2) + LT_C * 2 + 16 * (lane % 8),
                          rs + r8 * LT_R);
            }
        }
    };

    float m_ref = -INFINITY, l_part = 0.f;
    f32x4 o[LT_C / 16];
#pragma unroll
    for (int cb = 0; cb < LT_C / 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float c_log2 = p.scale_log2;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    int next_copy = 0;
    while (next_copy < min(n_tiles, LT_SLOTS - 1)) issue_tile(next_copy++);
    // the query fragments are complete before the loop (so the tile loop carries
    // no wait for them, which would also drain the copies in flight)
#pragma unroll
    for (int kk = 0; kk < LT_KK; ++kk) asm volatile("" ::"v"(qf[kk]));
    for (int t = 0; t < n_tiles; ++t) {
        // tile t landed for every wave (a wave issues 7 or 8 copies per tile, so
        // vmcnt(7k) leaves at most the k newer tiles in flight), and every wave
        // is done reading tile t-1, whose slot the copy of tile t+3 reuses.  A
        // bare barrier: a workgroup fence would also drain the newer copies.
        const int newer = next_copy - 1 - t;
        if (newer >= 2) __builtin_amdgcn_s_waitcnt(0x007E);        // vmcnt(14) lgkmcnt(0)
        else if (newer == 1) __builtin_amdgcn_s_waitcnt(0x0077);   // vmcnt(7) lgkmcnt(0)
        else __builtin_amdgcn_s_waitcnt(0x0070);                   // vmcnt(0) lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (next_copy < n_tiles) issue_tile(next_copy++);

        const __bf16 *cs = Cring[t % LT_SLOTS], *rs = Rring[t % LT_SLOTS];
        const int kb0 = k_begin + t * LT_BN;
        // S^T = C q~^T for the tile's 32 keys: A = 16 latent rows x 32 values
        f32x4 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const __bf16 *crow = cs + (16 * kb + r) * LT_CS + 8 * g;
            const __bf16 *rrow = rs + (16 * kb + r) * LT_R + 8 * g;
#pragma unroll
            for (int kk = 0; kk < LT_KK; ++kk) {
                const bf16x8 a = kk < LT_C / 32 ? *reinterpret_cast<const bf16x8 *>(crow + 32 * kk)
                                                : *reinterpret_cast<const bf16x8 *>(rrow + 32 * (kk - LT_C / 32));
                s[kb] = mfma16(a, qf[kk], kk == 0 ? zero4 : s[kb]);
            }
        }
        // keys past the chunk end are masked; row maximum in log2 units
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (kb0 + 16 * kb + 4 * g + e >= k_end) s[kb][e] = -INFINITY;
                mx = fmaxf(mx, s[kb][e]);
            }
        mx = group4_max(mx) * c_log2;
        const float m_new = fmaxf(m_ref, mx);
        if (__any(m_new > m_ref + RESCALE_LOG2)) {
            // lazy rescale: the reference only moves when a score exceeds it by 2^8
            const bool raise = m_new > m_ref + RESCALE_LOG2;
            const float alpha = raise ? fast_exp2(m_ref - m_new) : 1.f;
            m_ref = raise ? m_new : m_ref;
            l_part *= alpha;
#pragma unroll
            for (int cb = 0; cb < LT_C / 16; ++cb) o[cb] *= alpha;
        }
        const float mref = m_ref == -INFINITY ? 0.f : m_ref;
        uint32_t pw[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float pv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[e] = fast_exp2(fmaf(s[kb][e], c_log2, -mref));
            pw[2 * kb] = pack_bf16x2(pv[0], pv[1]);
            pw[2 * kb + 1] = pack_bf16x2(pv[2], pv[3]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) l_part = sum_bf16x2(pw[i], l_part);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, (u32x4{pw[0], pw[1], pw[2], pw[3]}));
        // o~^T += C^T P^T: A = 16 latent values x 32 keys from two transposing
        // reads: lane (r, g) receives C[4g + e][16cb + r] and C[16 + 4g + e][16cb + r]
        const __bf16 *vrd = cs + (4 * g + (r >> 2)) * LT_CS + 4 * (r & 3);
#pragma unroll
        for (int cb = 0; cb < LT_C / 16; ++cb) {
            const lt_s16x4 lo = lt_read_tr16(vrd + 16 * cb);
            const lt_s16x4 hi4 = lt_read_tr16(vrd + 16 * LT_CS + 16 * cb);
            const lt_s16x4 v8[2] = {lo, hi4};
            o[cb] = mfma16(__builtin_bit_cast(bf16x8, v8), pb, o[cb]);
        }
    }

    // partials of this chunk: m (log2 units), l and o~ per query head
    const float l_tot = group4_sum(l_part);
    if (!q_ok) return;
    const long pq = ((long)b * p.n_split + sp) * n_q + q_row;
    if (g == 0) {
        p.part_ml[2 * pq] = n_tiles > 0 ? m_ref : -INFINITY;
        p.part_ml[2 * pq + 1] = l_tot;
    }
    float *po = p.part_o + pq * LT_C + 4 * g;
#pragma unroll
    for (int cb = 0; cb < LT_C / 16; ++cb) *reinterpret_cast<f32x4 *>(po + 16 * cb) = o[cb];
}

// ---- 3. merge, combine in the latent space, up-project, gate.  Workgroup
// (KV head j, sequence b), 512 threads.
__global__ __launch_bounds__(LT_C) void latent_combine_kernel(LatentParams p) {
    __shared__ float dl[GROUP][LT_C];          // d~ of the 4 signal heads
    __shared__ float sc[HEADS][2];             // per head: merged reference and 1 / l
    const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int n_sig = p.n_kv * GROUP, n_q = n_sig + p.n_kv;
    // heads of group j: signal 4j .. 4j+3, noise n_sig + j
    if (tid < HEADS) {
        const int q = tid < GROUP ? GROUP * j + tid : n_sig + j;
        float m = -INFINITY;
        for (int s = 0; s < p.n_split; ++s) m = fmaxf(m, p.part_ml[2 * (((long)b * p.n_split + s) * n_q + q)]);
        float l = 0.f;
        for (int s = 0; s < p.n_split; ++s) {
            const long pq = ((long)b * p.n_split + s) * n_q + q;
            const float ms = p.part_ml[2 * pq];
            if (ms != -INFINITY) l += fast_exp2(ms - m) * p.part_ml[2 * pq + 1];
        }
        sc[tid][0] = m;
        sc[tid][1] = l > 0.f ? 1.f / l : 0.f;
    }
    __syncthreads();
    {
        const int c = tid;                     // latent value c of every head
        float acc[HEADS];
#pragma unroll
        for (int h = 0; h < HEADS; ++h) {
            const int q = h < GROUP ? GROUP * j + h : n_sig + j;
            float a = 0.f;
            for (int s = 0; s < p.n_split; ++s) {
                const long pq = ((long)b * p.n_split + s) * n_q + q;
                const float ms = p.part_ml[2 * pq];
                if (ms != -INFINITY) a += fast_exp2(ms - sc[h][0]) * p.part_o[pq * LT_C + c];
            }
            acc[h] = a * sc[h][1];
        }
        const long hrow = (long)b * n_sig + GROUP * j;
#pragma unroll
        for (int h = 0; h < GROUP; ++h) dl[h][c] = fmaf(-(float)p.lam[hrow + h], acc[GROUP], acc[h]);
    }
    __syncthreads();
    // D[h][d] = sum_c W_uv[j][d][c] d~[h][c]: thread (h, d) for h = tid / 128
    const int h = tid / D_V, d = tid % D_V;
    const __bf16 *w = p.wuv + ((long)j * D_V + d) * LT_C;
    float acc = 0.f;
    for (int c = 0; c < LT_C; c += 8) {
        const u32x4 wv = ldg16(w + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fmaf(bf16_lo(wv[i]), dl[h][c + 2 * i], acc);
            acc = fmaf(bf16_hi(wv[i]), dl[h][c + 2 * i + 1], acc);
        }
    }
    const long orow = (long)b * n_sig + GROUP * j + h;
    p.out[orow * D_V + d] = (__bf16)((float)p.gate[orow * D_V + d] * acc);
}

int latent_splits(int max_seqlen_k, int window) {
    const long vis = window > 0 ? (long)std::min(max_seqlen_k, window) : (long)max_seqlen_k;
    const long n = (vis + LT_CHUNK - 1) / LT_CHUNK;
    return (int)std::max(1L, std::min(n, 4096L));
}

size_t latent_workspace_bytes(int B, int n_kv, int n_split) {
    const size_t n_q = (size_t)n_kv * HEADS;
    const size_t qt = ((size_t)B * n_q * LT_ROW * 2 + 255) & ~(size_t)255;
    const size_t ml = ((size_t)B * n_split * n_q * 2 * sizeof(float) + 255) & ~(size_t)255;
    return qt + ml + (size_t)B * n_split * n_q * LT_C * sizeof(float);
}

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
    const size_t qt = ((size_t)B * n_q * LT_ROW * 2 + 255) & ~(size_t)255;
    const size_t ml = ((size_t)B * n_split * n_q * 2 * sizeof(float) + 255) & ~(size_t)255;
    p.qt = reinterpret_cast<__bf16 *>(ws);
    p.part_ml = reinterpret_cast<float *>(ws + qt);
    p.part_o = reinterpret_cast<float *>(ws + qt + ml);
    p.B = B;
    p.n_kv = n_kv;
    p.n_split = n_split;
    p.window = window;
    p.scale_log2 = scale * LOG2E;
    hipLaunchKernelGGL(latent_absorb_kernel, dim3(n_kv, (B + LT_ABS_SEQ - 1) / LT_ABS_SEQ), dim3(LT_C), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_hg = (int)((n_q + LT_HEADS_PER_WG - 1) / LT_HEADS_PER_WG);
    hipLaunchKernelGGL(latent_split_kernel, dim3(n_split, B, n_hg), dim3(LT_THREADS), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(latent_combine_kernel, dim3(n_kv, B), dim3(LT_C), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdla
