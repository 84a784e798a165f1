// gdn_decode.hip -- decode steps of the Gated DeltaNet mixer on gfx950.
//
// T new tokens per sequence, T = 1 for an ordinary step ("How Qwen3.5 works"
// §13.3: each linear layer shifts its conv state and takes one recurrent step
// per token).  A step is bound by HBM: every value head's 128x128 fp32 state
// (64 KiB) is read once and written once in place, 0.85 FLOP per byte.  With
// T > 1 (verifying draft tokens, "Qwen3.5-4B architecture" on MTP: propose
// tokens, check them in one forward pass) the state stays in registers across
// the T tokens and, when asked, the state and conv window after each token but
// the last are written as snapshots, so that the caller can roll back to any
// accepted prefix ("How Qwen3.5 works" §13.5: a recurrent state cannot be
// rewound, rollback needs snapshots).
//
// Work split: one workgroup per (sequence b, key head kh).  It owns the conv
// channels of that key head's q and k and of its r = Hv/Hk value heads, so
// the in-place conv-window shift has exactly one writer.  It then walks the r
// value heads; for each, 256 threads hold the 128x128 state in registers
// (thread = 4 value columns x 16 key rows, float4 loads: a wave reads two
// consecutive 512-byte rows per instruction), reduce S^T k and S^T q in one
// pass, and write S' = a S + k d^T.
//
// Read-out identity: with S' = a S + k d^T, o = S'^T q = a (S^T q) + (q.k) d,
// so both reductions come from the single read of S.  This follows from the
// decay -> predict -> correct -> read order of "How Qwen3.5 works" §9.6.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kD = 128;

struct DecodeArgs {
    const uint16_t *q, *k, *v, *z, *conv_w, *norm_w;
    const float *g, *beta;       // or the gate logits a, b when A_log is set
    const float *A_log, *dt_bias;
    float *state;
    uint16_t *conv_state, *o;
    float *state_snaps;        // [T-1][B][Hv][128][128] or nullptr
    uint16_t *conv_snaps;      // [T-1][B][3][Cc] or nullptr
    int B, T, Hk, Hv, r, Cc, conv, norm;
    float eps_l2, eps_norm;
};

constexpr int kMaxTokens = kMaxDecodeTokens;

__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    const int tid = threadIdx.x;
    const int b = blockIdx.x / a.Hk;
    const int kh = blockIdx.x % a.Hk;
    const int r = a.r, T = a.T;
    const int nu = 2 * kD + kD * r;  // conv outputs of one token

    // sU: conv output, per token, of this key head's q (0..127), k (128..255)
    // and the r value heads' v (256 + 128*hr + j).
    extern __shared__ float smem[];
    float *sU = smem;                   // [T][nu]
    float *sQn = sU + T * nu;           // [T][128] normalised q (incl. 1/sqrt(128))
    float *sKn = sQn + T * kD;          // [T][128] normalised k
    float *sRed = sKn + T * kD;         // [4 waves][2][128] partial sums
    float *sD = sRed + 4 * 2 * kD;      // correction d [128]
    float *sQK = sD + kD;               // [T] q^.k^
    float *sMisc = sQK + kMaxTokens;    // [0..1] norm partials

    // ---- 1. conv window shift + conv + SiLU on the owned channels, every token
    const int n_items = nu / 8;
    for (int it = tid; it < n_items; it += kThreads) {
        const uint16_t *xp;
        size_t xstride;  // elements from one token's row to the next
        int c;           // conv channel
        if (it < 16) {
            c = kh * kD + it * 8;
            xp = a.q + ((size_t)b * T * a.Hk + kh) * kD + it * 8;
            xstride = (size_t)a.Hk * kD;
        } else if (it < 32) {
            c = a.Hk * kD + kh * kD + (it - 16) * 8;
            xp = a.k + ((size_t)b * T * a.Hk + kh) * kD + (it - 16) * 8;
            xstride = (size_t)a.Hk * kD;
        } else {
            const int hr = (it - 32) >> 4, j8 = (it - 32) & 15;
            const int h = kh * r + hr;
            c = 2 * a.Hk * kD + h * kD + j8 * 8;
            xp = a.v + ((size_t)b * T * a.Hv + h) * kD + j8 * 8;
            xstride = (size_t)a.Hv * kD;
        }
        // raw inputs in time order: the three stored ones, then the T new tokens
        uint4 raw[3 + kMaxTokens];
#pragma unroll
        for (int t = 0; t < kMaxTokens; ++t)
            if (t < T) raw[3 + t] = *reinterpret_cast<const uint4 *>(xp + t * xstride);
        if (a.conv) {
            uint16_t *cs = a.conv_state + (size_t)b * 3 * a.Cc + c;
#pragma unroll
            for (int s = 0; s < 3; ++s) raw[s] = *reinterpret_cast<const uint4 *>(cs + s * a.Cc);
            const uint4 *wp = reinterpret_cast<const uint4 *>(a.conv_w + (size_t)c * 4);
            float w[32];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float tmp[8];
                unpack_bf16x8(wp[i], tmp);
#pragma unroll
                for (int e = 0; e < 8; ++e) w[8 * i + e] = tmp[e];
            }
            float x[4][8];  // a sliding window over raw[]
#pragma unroll
            for (int s = 0; s < 3; ++s) unpack_bf16x8(raw[s], x[s + 1]);
#pragma unroll
            for (int t = 0; t < kMaxTokens; ++t) {
                if (t < T) {
#pragma unroll
                    for (int s = 0; s < 3; ++s)
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[s][e] = x[s + 1][e];
                    unpack_bf16x8(raw[3 + t], x[3]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        // tap 3 multiplies the current token, tap 0 the one three before it
                        const float acc = w[4 * e + 0] * x[0][e] + w[4 * e + 1] * x[1][e] +
                                          w[4 * e + 2] * x[2][e] + w[4 * e + 3] * x[3][e];
                        sU[t * nu + it * 8 + e] = silu(acc);
                    }
                    // the window after token t: raw[t+1 .. t+3]; the last one replaces the stored window
                    uint16_t *dst = t == T - 1 ? cs
                                    : a.conv_snaps ? a.conv_snaps + ((size_t)t * a.B + b) * 3 * a.Cc + c
                                                   : nullptr;
                    if (dst) {
#pragma unroll
                        for (int s = 0; s < 3; ++s) *reinterpret_cast<uint4 *>(dst + s * a.Cc) = raw[t + 1 + s];
                    }
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < kMaxTokens; ++t) {
                if (t < T) {
                    float x[8];
                    unpack_bf16x8(raw[3 + t], x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) sU[t * nu + it * 8 + e] = x[e];
                }
            }
        }
    }
    __syncthreads();

    // ---- 2. per token: L2 norms of q and k and the raw q.k (one wave per task)
    const int wave = tid >> 6, lane = tid & 63;
    for (int task = wave; task < 3 * T; task += 4) {
        const int t = task / 3, kind = task % 3;  // 0: q, 1: k, 2: q.k
        const float *u = sU + t * nu;
        const float x0 = u[(kind == 1 ? kD : 0) + 2 * lane];
        const float x1 = u[(kind == 1 ? kD : 0) + 2 * lane + 1];
        if (kind < 2) {
            const float s = wave_sum(x0 * x0 + x1 * x1);
            float sc = 1.0f / sqrtf(s + a.eps_l2);
            if (kind == 0) sc *= 0.08838834764831845f;  // 1/sqrt(128)
            float *dst = (kind == 0 ? sQn : sKn) + t * kD;
            dst[2 * lane] = x0 * sc;
            dst[2 * lane + 1] = x1 * sc;
        } else {
            const float xq0 = x0, xq1 = x1;
            const float xk0 = u[kD + 2 * lane], xk1 = u[kD + 2 * lane + 1];
            const float sqk = wave_sum(xq0 * xk0 + xq1 * xk1);
            const float sq = wave_sum(xq0 * xq0 + xq1 * xq1), sk = wave_sum(xk0 * xk0 + xk1 * xk1);
            if (lane == 0)  // the raw q.k times both norms' scales (the same products as above)
                sQK[t] = sqk * ((1.0f / sqrtf(sq + a.eps_l2)) * 0.08838834764831845f) * (1.0f / sqrtf(sk + a.eps_l2));
        }
    }
    __syncthreads();

    // thread tile of the state: columns 4*jg..4*jg+3, rows rg + 8*m
    const int jg = tid & 31, rg = tid >> 5;

    for (int hr = 0; hr < r; ++hr) {
        const int h = kh * r + hr;
        const size_t hb = (size_t)b * a.Hv + h;
        float4 *Sp = reinterpret_cast<float4 *>(a.state + hb * kD * kD);
        float4 S[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) S[m] = Sp[(rg + 8 * m) * (kD / 4) + jg];
        for (int t = 0; t < T; ++t) {
            const size_t ht = ((size_t)b * T + t) * a.Hv + h;  // (sequence, token, head) row
            const float *qn = sQn + t * kD, *kn = sKn + t * kD;
            const float qk = sQK[t];
            float gl = a.g[ht], beta = a.beta[ht];
            if (a.A_log) {  // gates from their logits
                gl = gate_g(gl, a.A_log[h], a.dt_bias[h]);
                beta = gate_beta(beta);
            }
            const float alpha = __expf(gl);

            float pk[4] = {0, 0, 0, 0}, pq[4] = {0, 0, 0, 0};
    #pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float kv = kn[rg + 8 * m], qv = qn[rg + 8 * m];
                pk[0] += S[m].x * kv; pk[1] += S[m].y * kv; pk[2] += S[m].z * kv; pk[3] += S[m].w * kv;
                pq[0] += S[m].x * qv; pq[1] += S[m].y * qv; pq[2] += S[m].z * qv; pq[3] += S[m].w * qv;
            }
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
                pk[e] += __shfl_xor(pk[e], 32, 64);
                pq[e] += __shfl_xor(pq[e], 32, 64);
            }
            if (lane < 32) {
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sRed[(wave * 2 + 0) * kD + 4 * jg + e] = pk[e];
                    sRed[(wave * 2 + 1) * kD + 4 * jg + e] = pq[e];
                }
            }
            __syncthreads();

            float oj = 0.0f;
            if (tid < kD) {
                const int j = tid;
                const float PK = sRed[0 * kD + j] + sRed[2 * kD + j] + sRed[4 * kD + j] + sRed[6 * kD + j];
                const float PQ = sRed[1 * kD + j] + sRed[3 * kD + j] + sRed[5 * kD + j] + sRed[7 * kD + j];
                const float vj = sU[t * nu + 2 * kD + hr * kD + j];
                const float d = beta * (vj - alpha * PK);
                oj = alpha * PQ + qk * d;
                sD[j] = d;
                if (a.norm) {
                    const float ss = wave_sum(oj * oj);
                    if (lane == 0) sMisc[wave] = ss;
                }
            }
            __syncthreads();

            // S' = a S + k d^T: in place after the last token, as a snapshot after the others
            const float4 d4 = reinterpret_cast<const float4 *>(sD)[jg];
            float4 *dst = Sp;
            if (t < T - 1)
                dst = a.state_snaps ? reinterpret_cast<float4 *>(a.state_snaps + (((size_t)t * a.B + b) * a.Hv + h) * kD * kD)
                                    : nullptr;
    #pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float kv = kn[rg + 8 * m];
                float4 s = S[m];
                s.x = alpha * s.x + kv * d4.x;
                s.y = alpha * s.y + kv * d4.y;
                s.z = alpha * s.z + kv * d4.z;
                s.w = alpha * s.w + kv * d4.w;
                S[m] = s;
                if (dst) dst[(rg + 8 * m) * (kD / 4) + jg] = s;
            }

            if (tid < kD) {
                const int j = tid;
                float y = oj;
                if (a.norm) {
                    const float ms = (sMisc[0] + sMisc[1]) * (1.0f / kD);
                    const float rstd = 1.0f / sqrtf(ms + a.eps_norm);
                    const float zj = bf16_to_f32(a.z[ht * kD + j]);
                    y = bf16_to_f32(a.norm_w[j]) * (oj * rstd) * silu(zj);
                }
                a.o[ht * kD + j] = f32_to_bf16(y);
            }
            __syncthreads();  // sRed / sD / sMisc are reused by the next token or head
        }
    }
}

} // namespace

size_t decode_lds_bytes(int T, int r) {
    return sizeof(float) * ((size_t)T * (2 * kD + kD * r) + (size_t)2 * T * kD + 8 * kD + kD + kMaxTokens + 8);
}

int launch_decode(const DecodeParams &p, hipStream_t stream) {
    DecodeArgs a;
    a.q = p.q; a.k = p.k; a.v = p.v; a.z = p.z; a.conv_w = p.conv_w; a.norm_w = p.norm_w;
    a.g = p.g; a.beta = p.beta; a.A_log = p.A_log; a.dt_bias = p.dt_bias; a.state = p.state; a.conv_state = p.conv_state; a.o = p.o;
    a.state_snaps = p.state_snaps; a.conv_snaps = p.conv_snaps;
    a.B = p.B; a.T = p.T; a.Hk = p.Hk; a.Hv = p.Hv; a.r = p.Hv / p.Hk;
    a.Cc = 2 * p.Hk * kD + p.Hv * kD;
    a.conv = p.conv_width == 4; a.norm = p.norm;
    a.eps_l2 = p.eps_l2; a.eps_norm = p.eps_norm;
    if (p.T < 1 || p.T > kMaxTokens) return fail("decode: tokens per sequence out of range");
    const size_t lds = decode_lds_bytes(p.T, a.r);
    if (lds > 160 * 1024) return fail("decode: head ratio and token count need more LDS than a workgroup has");
    void *args[] = {&a};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(decode_kernel), dim3((unsigned)(p.B * p.Hk)),
                                         dim3(kThreads), args, lds, stream);
    return e == hipSuccess ? 0 : fail("hipLaunchKernel(decode_kernel)", e);
}

} // namespace gdn
