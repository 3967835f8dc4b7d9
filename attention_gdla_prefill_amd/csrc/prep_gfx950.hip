// prep_gfx950.hip -- the step ahead of the GDLA attention core, fused into
// one pass over the tokens:
//   - rotary position embedding of the 64-value rotary part of every query
//     head (in place) and of the decoupled rotary key, which is shared by all
//     KV heads and is written into the rotary part of each of them
//     (aitrends.kr, GDLA paragraph: the query path yields a content query and
//     a rotary query, the KV path a decoupled rotary key; head-dimension
//     paragraph: a 64-value rotary component, the rotary key shared by every
//     KV head);
//   - lambda_t = sigmoid(x_t W^lambda), one value per signal head (same page,
//     first GDLA paragraph);
//   - the sigmoid of the output gate's pre-activations (metalmedia, Table 1:
//     attention with output gating; the gate's projection is an ordinary
//     matmul done before this step).
// The rotation is the original rotary embedding on adjacent pairs
// (2i, 2i+1), turned counter-clockwise by pos * theta^(-2i/64); token t of
// every sequence sits at position pos0 + t.
//
// Blocks of PP_TOK = 16 consecutive tokens (of the flattened [B*T]), 4 waves
// per workgroup.  The step moves ~62 KB per token and does ~0.5 MFLOP of
// lambda per token, so it is bound by HBM; lambda runs on MFMA so that its
// 4096-long dot products stay off the critical path, and from LAM_WIDE_MIN_TOK
// tokens on it stages W^lambda in LDS for 64 tokens at a time, which keeps its
// re-reads of W^lambda from the L2 below those of x from HBM.
#include "gdla_device.h"
#include "gdla_launch.h"

namespace gdla {

constexpr int PP_TOK = 16;            // tokens per workgroup (the MFMA M dimension of lambda)
constexpr int PP_THREADS = 256;
constexpr int PP_ROT = 64;            // rotary values per head, the last 64 of D_QK
constexpr int PP_PAIRS = PP_ROT / 2;

struct PrepParams {
    __bf16 *qs, *qn, *k;                  // in place / rotary part written
    const __bf16 *k_rope, *x, *w_lambda, *gate_pre;
    __bf16 *lam, *gate;
    long n_tok;                           // B * T
    int lam_wide;                         // lambda by LAM_TOK-token workgroups (else 16-token ones)
    int T, n_kv, d_model, pos0;
    double theta;
};

// Workgroup (16-token block, job): job 0 = lambda, job 1 = rotary
// embedding, jobs 2 .. 1+PP_GATE_PARTS = one part each of the gate, so that
// the memory streams of a block run side by side on different CUs.  In the
// wide form of lambda, job-0 workgroup x takes tokens 64x .. 64x+63, and those
// past the end return at once.
constexpr int PP_GATE_PARTS = 4;
constexpr int PP_JOBS = 2 + PP_GATE_PARTS;
constexpr int PP_HB = 4;              // head blocks of 16 per lambda pass (64 heads)
constexpr int LAM_TOK = 64;           // tokens per lambda workgroup (16 per wave)
constexpr int LAM_KC = 64;            // d_model values per staged W^lambda chunk
constexpr int LAM_ROW = 2 * LAM_KC + 16;  // LDS bytes per head row of a chunk (16 padding)
constexpr int LAM_BUF = 64 * LAM_ROW;     // one chunk for 64 heads
// From this many tokens on, lambda takes the wide form: it then has enough
// workgroups to fill the chip, and it reads W^lambda a quarter as often.
// Below it, the 16-token form's four times as many workgroups finish sooner.
constexpr long LAM_WIDE_MIN_TOK = 8192;
static_assert(2 * LAM_BUF >= (int)sizeof(float2) * PP_TOK * PP_PAIRS, "LDS union too small");
static_assert(2 * LAM_BUF >= (int)sizeof(float) * 4 * PP_TOK * PP_HB * 16, "LDS union too small");
constexpr int PP_BATCH = 4;           // rotary tasks / gate chunks per thread in flight

__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, float2 c) {
    const float x0 = bf16_lo(w), x1 = bf16_hi(w);
    return pack_bf16x2(x0 * c.x - x1 * c.y, x0 * c.y + x1 * c.x);
}

__global__ __launch_bounds__(PP_THREADS) void prep_kernel(PrepParams p) {
    // lambda's two W^lambda chunks, or (cos, sin) of every (token, pair) of the block
    __shared__ __align__(16) unsigned char smem[2 * LAM_BUF];
    float2 (*cs)[PP_PAIRS] = reinterpret_cast<float2 (*)[PP_PAIRS]>(smem);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, job = blockIdx.y;
    const long tok0 = (long)blockIdx.x * PP_TOK;
    const int n_tok_blk = (int)min((long)PP_TOK, p.n_tok - tok0);
    const int n_sig = p.n_kv * GROUP, n_qh = n_sig + p.n_kv;

    if (job == 0 && !p.lam_wide) {
        float (*red)[PP_TOK][PP_HB * 16] = reinterpret_cast<float (*)[PP_TOK][PP_HB * 16]>(smem);
        // ---- lambda = sigmoid(x W^lambda^T).  Wave w takes a quarter of the
        // d_model/32 steps for 64 heads at a time (4 MFMA chains).  A = x rows
        // (lane (r, g): token r, values 8g..8g+7 of a 32-value step), B =
        // W^lambda rows (lane (r, g): head r, the same 8 values); the four
        // partial sums meet in LDS.
        const int r = lane & 15, g = lane >> 4;
        const long tok = tok0 + r;
        const bool t_ok = r < n_tok_blk;
        const int n_steps = p.d_model / 32;
        const int s_lo = wave * n_steps / 4, s_hi = (wave + 1) * n_steps / 4;
        const __bf16 *xa = p.x + (t_ok ? tok : tok0) * p.d_model + 8 * g;
        const u32x4 z = {0, 0, 0, 0};
        for (int h0 = 0; h0 < n_sig; h0 += PP_HB * 16) {
            const __bf16 *wb[PP_HB];
            bool h_ok[PP_HB];
#pragma unroll
            for (int hb = 0; hb < PP_HB; ++hb) {
                h_ok[hb] = h0 + 16 * hb + r < n_sig;
                wb[hb] = p.w_lambda + (long)(h_ok[hb] ? h0 + 16 * hb + r : 0) * p.d_model + 8 * g;
            }
            f32x4 acc[PP_HB];
#pragma unroll
            for (int hb = 0; hb < PP_HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s0 = s_lo; s0 < s_hi; s0 += 4) {
                // four steps per round: their 20 loads are issued together
                bf16x8 a[4], bw[4][PP_HB];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bool in = s0 + s < s_hi;
                    a[s] = __builtin_bit_cast(bf16x8, (t_ok && in) ? ldg16(xa + 32 * (s0 + s)) : z);
#pragma unroll
                    for (int hb = 0; hb < PP_HB; ++hb)
                        bw[s][hb] = __builtin_bit_cast(bf16x8, (h_ok[hb] && in) ? ldg16(wb[hb] + 32 * (s0 + s)) : z);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int hb = 0; hb < PP_HB; ++hb) acc[hb] = mfma16(a[s], bw[s][hb], acc[hb]);
            }
            // lane (r, g) holds tokens 4g..4g+3 of head h0 + 16hb + r
#pragma unroll
            for (int hb = 0; hb < PP_HB; ++hb)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[wave][4 * g + e][16 * hb + r] = acc[hb][e];
            __syncthreads();
            for (int i = tid; i < PP_TOK * PP_HB * 16; i += PP_THREADS) {
                const int tl = i / (PP_HB * 16), hh = i % (PP_HB * 16);
                if (tl < n_tok_blk && h0 + hh < n_sig) {
                    const float zz = red[0][tl][hh] + red[1][tl][hh] + red[2][tl][hh] + red[3][tl][hh];
                    p.lam[(tok0 + tl) * n_sig + h0 + hh] = (__bf16)(1.f / (1.f + __expf(-zz)));
                }
            }
            __syncthreads();
        }
    } else if (job == 0) {
        // ---- lambda = sigmoid(x W^lambda^T) for LAM_TOK tokens: wave w owns
        // tokens 16w..16w+15 and 64 heads at a time (4 MFMA chains).  The
        // W^lambda chunk of LAM_KC values is staged in LDS once for the 4
        // waves (double-buffered; the loads of W^lambda and of the x rows are
        // requested two chunks ahead of their products), so W^lambda is read
        // once per LAM_TOK tokens.  A = x
        // rows (lane (r, g): token r, values 8g..8g+7 of a 32-value step), B =
        // W^lambda rows from LDS (lane (r, g): head r, the same values).
        const long lt0 = (long)blockIdx.x * LAM_TOK;
        if (lt0 >= p.n_tok) return;
        const int r = lane & 15, g = lane >> 4;
        const long tok = lt0 + 16 * wave + r;
        const bool t_ok = tok < p.n_tok;
        const __bf16 *xa = p.x + (t_ok ? tok : 0) * p.d_model + 8 * g;
        const int n_ch = (p.d_model + LAM_KC - 1) / LAM_KC;
        const u32x4 z = {0, 0, 0, 0};
        for (int h0 = 0; h0 < n_sig; h0 += 64) {
            // this thread's share of a W^lambda chunk: 16-byte pieces tid and tid + 256
            auto load_w = [&](int c, u32x4 (&w)[2]) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int i = tid + PP_THREADS * u, hh = i >> 3, k = c * LAM_KC + 8 * (i & 7);
                    w[u] = (c < n_ch && h0 + hh < n_sig && k < p.d_model)
                               ? ldg16(p.w_lambda + (long)(h0 + hh) * p.d_model + k) : z;
                }
            };
            auto store_w = [&](int c, const u32x4 (&w)[2]) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int i = tid + PP_THREADS * u;
                    *reinterpret_cast<u32x4 *>(smem + (c & 1) * LAM_BUF + (i >> 3) * LAM_ROW + 16 * (i & 7)) = w[u];
                }
            };
            auto load_x = [&](int c, u32x4 (&a)[2]) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int k = c * LAM_KC + 32 * s;
                    a[s] = (t_ok && c < n_ch && k < p.d_model) ? ldg16(xa + k) : z;
                }
            };
            f32x4 acc[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
            u32x4 wn[2], w2[2], xc[2], xn[2], x2[2];
            load_w(0, wn);
            load_x(0, xc);
            load_x(1, xn);
            store_w(0, wn);
            load_w(1, wn);
            __syncthreads();
            for (int c = 0; c < n_ch; ++c) {
                load_w(c + 2, w2);
                load_x(c + 2, x2);
                const unsigned char *buf = smem + (c & 1) * LAM_BUF;
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int hb = 0; hb < 4; ++hb) {
                        const u32x4 b = *reinterpret_cast<const u32x4 *>(buf + (16 * hb + r) * LAM_ROW + 64 * s + 16 * g);
                        acc[hb] = mfma16(__builtin_bit_cast(bf16x8, xc[s]), __builtin_bit_cast(bf16x8, b), acc[hb]);
                    }
                store_w(c + 1, wn);
                __syncthreads();
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    wn[u] = w2[u];
                    xc[u] = xn[u];
                    xn[u] = x2[u];
                }
            }
            // lane (r, g) holds tokens 4g..4g+3 (of the wave's 16) of head h0 + 16hb + r
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const long t = lt0 + 16 * wave + 4 * g + e;
                    const int h = h0 + 16 * hb + r;
                    if (t < p.n_tok && h < n_sig)
                        p.lam[t * n_sig + h] = (__bf16)(1.f / (1.f + __expf(-acc[hb][e])));
                }
        }
    } else if (job == 1) {
        // ---- angles: fp64 from position and frequency to sine and cosine (a
        // position of 2^18 times a frequency of 1 keeps ~1e-11 rad), fp32 after
        for (int i = tid; i < PP_TOK * PP_PAIRS; i += PP_THREADS) {
            const int tl = i / PP_PAIRS, pr = i % PP_PAIRS;
            const double pos = (double)(p.pos0 + (tl < n_tok_blk ? (tok0 + tl) % p.T : 0));
            const double ang = pos * pow(p.theta, -2.0 * pr / PP_ROT);
            cs[tl][pr] = make_float2((float)cos(ang), (float)sin(ang));
        }
        __syncthreads();
        // ---- rotary parts of the query heads, in place: a task is one 16-byte
        // chunk (4 pairs) of one head of one token; 8 chunks per head
        // PP_BATCH tasks per thread are loaded before any is stored (the
        // compiler cannot move a load above a store that may alias it), so
        // their memory latencies overlap; a task past the end re-reads the last
        // task's chunk and is not stored.
        const int n_tasks = n_tok_blk * n_qh * 8;
        for (int i0 = tid; i0 < n_tasks; i0 += PP_BATCH * PP_THREADS) {
            u32x4 *addr[PP_BATCH];
            u32x4 w[PP_BATCH];
            int tls[PP_BATCH], chs[PP_BATCH];
#pragma unroll
            for (int u = 0; u < PP_BATCH; ++u) {
                const int i = min(i0 + u * PP_THREADS, n_tasks - 1);
                const int tl = i / (n_qh * 8), rem = i % (n_qh * 8), h = rem / 8, ch = rem % 8;
                const long tok = tok0 + tl;
                __bf16 *row = h < n_sig ? p.qs + (tok * n_sig + h) * D_QK
                                        : p.qn + (tok * p.n_kv + (h - n_sig)) * D_QK;
                addr[u] = reinterpret_cast<u32x4 *>(row + (D_QK - PP_ROT) + 8 * ch);
                tls[u] = tl;
                chs[u] = ch;
                w[u] = *addr[u];
            }
#pragma unroll
            for (int u = 0; u < PP_BATCH; ++u) {
                if (i0 + u * PP_THREADS >= n_tasks) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[u][e] = rotate_pair(w[u][e], cs[tls[u]][4 * chs[u] + e]);
                *addr[u] = w[u];
            }
        }
        // ---- the shared rotary key: rotated once per chunk, written to every KV head
        for (int i = tid; i < n_tok_blk * 8; i += PP_THREADS) {
            const int tl = i / 8, ch = i % 8;
            const long tok = tok0 + tl;
            u32x4 w = *reinterpret_cast<const u32x4 *>(p.k_rope + tok * PP_ROT + 8 * ch);
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = rotate_pair(w[e], cs[tl][4 * ch + e]);
            for (int j = 0; j < p.n_kv; ++j)
                *reinterpret_cast<u32x4 *>(p.k + (tok * p.n_kv + j) * D_QK + (D_QK - PP_ROT) + 8 * ch) = w;
        }
    } else {
        // ---- gate = sigmoid(pre-activation): part job-2 of the block's 16-byte chunks
        const long per_tok = (long)n_sig * D_V / 8;
        const long n_chunks = n_tok_blk * per_tok;
        const int part = job - 2;
        const long lo = tok0 * per_tok + n_chunks * part / PP_GATE_PARTS;
        const long hi = tok0 * per_tok + n_chunks * (part + 1) / PP_GATE_PARTS;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(p.gate_pre);
        u32x4 *dst = reinterpret_cast<u32x4 *>(p.gate);
        // PP_BATCH chunks per thread in flight (loads first, as above)
        for (long c0 = lo + tid; c0 < hi; c0 += PP_BATCH * PP_THREADS) {
            u32x4 w[PP_BATCH];
#pragma unroll
            for (int u = 0; u < PP_BATCH; ++u) w[u] = src[min(c0 + (long)u * PP_THREADS, hi - 1)];
#pragma unroll
            for (int u = 0; u < PP_BATCH; ++u) {
                if (c0 + (long)u * PP_THREADS >= hi) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float z0 = bf16_lo(w[u][e]), z1 = bf16_hi(w[u][e]);
                    w[u][e] = pack_bf16x2(1.f / (1.f + __expf(-z0)), 1.f / (1.f + __expf(-z1)));
                }
                dst[c0 + (long)u * PP_THREADS] = w[u];
            }
        }
    }
}

long prep_grid_blocks(long n_tok) { return (n_tok + PP_TOK - 1) / PP_TOK; }

hipError_t launch_prep(void *q_signal, void *q_noise, const void *k_rope, void *k, const void *x,
                       const void *w_lambda, void *lambda_out, const void *gate_pre, void *gate_out,
                       int B, int T, int n_kv, int d_model, int pos0, float rope_theta, hipStream_t stream) {
    PrepParams p;
    p.qs = static_cast<__bf16 *>(q_signal);
    p.qn = static_cast<__bf16 *>(q_noise);
    p.k = static_cast<__bf16 *>(k);
    p.k_rope = static_cast<const __bf16 *>(k_rope);
    p.x = static_cast<const __bf16 *>(x);
    p.w_lambda = static_cast<const __bf16 *>(w_lambda);
    p.gate_pre = static_cast<const __bf16 *>(gate_pre);
    p.lam = static_cast<__bf16 *>(lambda_out);
    p.gate = static_cast<__bf16 *>(gate_out);
    p.n_tok = (long)B * T;
    p.T = T;
    p.n_kv = n_kv;
    p.d_model = d_model;
    p.pos0 = pos0;
    p.theta = (double)rope_theta;
    p.lam_wide = p.n_tok >= LAM_WIDE_MIN_TOK;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)prep_grid_blocks(p.n_tok), PP_JOBS), dim3(PP_THREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdla
