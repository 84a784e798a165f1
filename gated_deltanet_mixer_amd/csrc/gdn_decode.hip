// gdn_decode.hip -- one decode step of the Gated DeltaNet mixer on gfx950.
//
// One new token per sequence ("How Qwen3.5 works" §13.3: each linear layer
// shifts its conv state and takes one recurrent step).  The step is bound by
// HBM: every value head's 128x128 fp32 state (64 KiB) is read once and
// written once in place, 0.85 FLOP per byte.
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
    int B, Hk, Hv, r, Cc, conv, norm;
    float eps_l2, eps_norm;
};

__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    const int tid = threadIdx.x;
    const int b = blockIdx.x / a.Hk;
    const int kh = blockIdx.x % a.Hk;
    const int r = a.r;

    // sU: conv output of this key head's q (0..127), k (128..255) and the r
    // value heads' v (256 + 128*hr + j).  At most 256 + 128*r floats.
    extern __shared__ float smem[];
    float *sU = smem;
    float *sQn = sU + 2 * kD + kD * r;  // normalised q (incl. 1/sqrt(128))
    float *sKn = sQn + kD;              // normalised k
    float *sRed = sKn + kD;             // [4 waves][2][128] partial sums
    float *sD = sRed + 4 * 2 * kD;      // correction d [128]
    float *sMisc = sD + kD;             // [0]=q scale [1]=k scale [2]=q.k raw [3..4]=norm partials

    // ---- 1. conv window shift + conv + SiLU on the owned channels
    const int n_items = (2 * kD + r * kD) / 8;
    for (int it = tid; it < n_items; it += kThreads) {
        const uint16_t *xp;
        int c;  // conv channel
        if (it < 16) {
            c = kh * kD + it * 8;
            xp = a.q + ((size_t)b * a.Hk + kh) * kD + it * 8;
        } else if (it < 32) {
            c = a.Hk * kD + kh * kD + (it - 16) * 8;
            xp = a.k + ((size_t)b * a.Hk + kh) * kD + (it - 16) * 8;
        } else {
            const int hr = (it - 32) >> 4, j8 = (it - 32) & 15;
            const int h = kh * r + hr;
            c = 2 * a.Hk * kD + h * kD + j8 * 8;
            xp = a.v + ((size_t)b * a.Hv + h) * kD + j8 * 8;
        }
        const uint4 xr = *reinterpret_cast<const uint4 *>(xp);
        float x[8], u[8];
        unpack_bf16x8(xr, x);
        if (a.conv) {
            uint16_t *cs = a.conv_state + (size_t)b * 3 * a.Cc + c;
            const uint4 s0r = *reinterpret_cast<const uint4 *>(cs);
            const uint4 s1r = *reinterpret_cast<const uint4 *>(cs + a.Cc);
            const uint4 s2r = *reinterpret_cast<const uint4 *>(cs + 2 * a.Cc);
            const uint4 *wp = reinterpret_cast<const uint4 *>(a.conv_w + (size_t)c * 4);
            float s0[8], s1[8], s2[8], w[32];
            unpack_bf16x8(s0r, s0);
            unpack_bf16x8(s1r, s1);
            unpack_bf16x8(s2r, s2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float tmp[8];
                unpack_bf16x8(wp[i], tmp);
#pragma unroll
                for (int e = 0; e < 8; ++e) w[8 * i + e] = tmp[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // tap 3 multiplies the current token, tap 0 the oldest stored one
                const float acc = w[4 * e + 0] * s0[e] + w[4 * e + 1] * s1[e] +
                                  w[4 * e + 2] * s2[e] + w[4 * e + 3] * x[e];
                u[e] = silu(acc);
            }
            // shift the window: oldest out, current token in
            *reinterpret_cast<uint4 *>(cs) = s1r;
            *reinterpret_cast<uint4 *>(cs + a.Cc) = s2r;
            *reinterpret_cast<uint4 *>(cs + 2 * a.Cc) = xr;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = x[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) sU[it * 8 + e] = u[e];
    }
    __syncthreads();

    // ---- 2. L2 norms of q and k (waves 0, 1) and the raw q.k (wave 2)
    const int wave = tid >> 6, lane = tid & 63;
    if (wave < 3) {
        const float x0 = sU[(wave == 1 ? kD : 0) + 2 * lane];
        const float x1 = sU[(wave == 1 ? kD : 0) + 2 * lane + 1];
        float s;
        if (wave == 2)
            s = wave_sum(x0 * sU[kD + 2 * lane] + x1 * sU[kD + 2 * lane + 1]);
        else
            s = wave_sum(x0 * x0 + x1 * x1);
        if (wave < 2) {
            float sc = 1.0f / sqrtf(s + a.eps_l2);
            if (wave == 0) sc *= 0.08838834764831845f;  // 1/sqrt(128)
            float *dst = wave == 0 ? sQn : sKn;
            dst[2 * lane] = x0 * sc;
            dst[2 * lane + 1] = x1 * sc;
            if (lane == 0) sMisc[wave] = sc;
        } else if (lane == 0) {
            sMisc[2] = s;
        }
    }
    __syncthreads();
    const float qk = sMisc[2] * sMisc[0] * sMisc[1];

    // thread tile of the state: columns 4*jg..4*jg+3, rows rg + 8*m
    const int jg = tid & 31, rg = tid >> 5;

    for (int hr = 0; hr < r; ++hr) {
        const int h = kh * r + hr;
        const size_t hb = (size_t)b * a.Hv + h;
        float4 *Sp = reinterpret_cast<float4 *>(a.state + hb * kD * kD);
        float4 S[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) S[m] = Sp[(rg + 8 * m) * (kD / 4) + jg];
        float gl = a.g[hb], beta = a.beta[hb];
        if (a.A_log) {  // gates from their logits
            gl = gate_g(gl, a.A_log[h], a.dt_bias[h]);
            beta = gate_beta(beta);
        }
        const float alpha = __expf(gl);

        float pk[4] = {0, 0, 0, 0}, pq[4] = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float kv = sKn[rg + 8 * m], qv = sQn[rg + 8 * m];
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
            const float vj = sU[2 * kD + hr * kD + j];
            const float d = beta * (vj - alpha * PK);
            oj = alpha * PQ + qk * d;
            sD[j] = d;
            if (a.norm) {
                const float ss = wave_sum(oj * oj);
                if (lane == 0) sMisc[3 + wave] = ss;
            }
        }
        __syncthreads();

        // S' = a S + k d^T, written in place
        const float4 d4 = reinterpret_cast<const float4 *>(sD)[jg];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float kv = sKn[rg + 8 * m];
            float4 s = S[m];
            s.x = alpha * s.x + kv * d4.x;
            s.y = alpha * s.y + kv * d4.y;
            s.z = alpha * s.z + kv * d4.z;
            s.w = alpha * s.w + kv * d4.w;
            Sp[(rg + 8 * m) * (kD / 4) + jg] = s;
        }

        if (tid < kD) {
            const int j = tid;
            float y = oj;
            if (a.norm) {
                const float ms = (sMisc[3] + sMisc[4]) * (1.0f / kD);
                const float rstd = 1.0f / sqrtf(ms + a.eps_norm);
                const float zj = bf16_to_f32(a.z[hb * kD + j]);
                y = bf16_to_f32(a.norm_w[j]) * (oj * rstd) * silu(zj);
            }
            a.o[hb * kD + j] = f32_to_bf16(y);
        }
        __syncthreads();  // sRed / sD / sMisc are reused by the next head
    }
}

} // namespace

int launch_decode(const DecodeParams &p, hipStream_t stream) {
    DecodeArgs a;
    a.q = p.q; a.k = p.k; a.v = p.v; a.z = p.z; a.conv_w = p.conv_w; a.norm_w = p.norm_w;
    a.g = p.g; a.beta = p.beta; a.A_log = p.A_log; a.dt_bias = p.dt_bias; a.state = p.state; a.conv_state = p.conv_state; a.o = p.o;
    a.B = p.B; a.Hk = p.Hk; a.Hv = p.Hv; a.r = p.Hv / p.Hk;
    a.Cc = 2 * p.Hk * kD + p.Hv * kD;
    a.conv = p.conv_width == 4; a.norm = p.norm;
    a.eps_l2 = p.eps_l2; a.eps_norm = p.eps_norm;
    const size_t lds = sizeof(float) * ((size_t)2 * kD + (size_t)kD * a.r + 2 * kD + 8 * kD + kD + 8);
    if (lds > 160 * 1024) return fail("decode: head ratio needs more LDS than a workgroup has");
    void *args[] = {&a};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(decode_kernel), dim3((unsigned)(p.B * p.Hk)),
                                         dim3(kThreads), args, lds, stream);
    return e == hipSuccess ? 0 : fail("hipLaunchKernel(decode_kernel)", e);
}

} // namespace gdn
