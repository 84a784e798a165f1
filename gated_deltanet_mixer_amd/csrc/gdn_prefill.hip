// gdn_prefill.hip -- chunked prefill of the Gated DeltaNet mixer on gfx950.
//
// Math ("How Qwen3.5 works" §9.11, the unit lower-triangular chunk form of
// the §9.6 recurrence).  Per chunk of C = 64 tokens with start state S
// (K-major, 128 x 128 fp32), cumulative log-decay G_i = sum_{s<=i} g_s and
// R_ij = exp(G_i - G_j) (j <= i):
//   A     = I + L,  L = strictly-lower(beta_i (k_i . k_j) R_ij)
//   T     = A^{-1}                       (unit lower triangular)
//   X     = V - diag(e^G) K S            (the page's U - W S with W = T diag(beta e^G) K
//   Delta = T diag(beta) X                and U = T diag(beta) V, factored through T)
//   O     = diag(e^G) Q S + ((Q K^T) o R) Delta
//   S'    = e^{G_C} S + K^T diag(e^{G_C - G_j}) Delta
// followed by the gated RMSNorm of each output row (model spec node gdn.norm).
//
// Kernels.
//  qk_prep_kernel   conv + SiLU + L2 norm (+ 1/sqrt(128) on q) of every
//                   (token, key head) q/k row, once, into an fp16 workspace.
//                   Shared by the r value heads and the value slices reading
//                   that key head; doing it in the chain kernel would repeat
//                   this VALU-heavy step r * nslice times.
//  chain_kernel<BV> one workgroup per (sequence, value head, slice of BV value
//                   columns); columns of the state evolve independently, so a
//                   head splits into 128/BV slices spread over CUs.  The loop
//                   over chunks is the only sequential dependency.  All
//                   contractions run on fp16 MFMA (v_mfma_f32_16x16x32_f16)
//                   with fp32 accumulation; the state is carried in fp32
//                   accumulators across chunks.  The gated RMSNorm needs all
//                   128 columns of a row: slices publish per-row sums of
//                   squares as tagged 64-bit words (value | chunk tag) and read
//                   their siblings' one chunk later.  Siblings are co-resident
//                   (cooperative launch), every wait is bounded.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kD = 128;        // head width
constexpr int kC = 64;         // chunk length
constexpr int kThreads = 256;  // 4 waves
constexpr int kRing = 4;       // chunks of partial sums kept per slice
constexpr int kCUs = 256;      // MI355X compute units: sizing of the value slicing
constexpr uint32_t kSpinLimit = 1u << 20;  // bound of every cross-workgroup wait (~0.3 s)

// LDS pitches (in elements) chosen so that 16-row MFMA fragment reads hit
// distinct banks.
constexpr int P128 = kD + 8;   // fp16 rows of 128
constexpr int P64 = kC + 8;    // fp16 rows of 64
constexpr int PL = kC + 4;     // fp32 rows of 64
constexpr int PTD = 20;        // fp32 rows of a 16x16 block

// ------------------------------------------------------------------------
// q/k preparation: u = silu(conv(x)), x^ = u / sqrt(sum u^2 + eps) (* 1/sqrt(128) for q)
// ------------------------------------------------------------------------

struct PrepArgs {
    const uint16_t *q, *k, *conv_w, *conv_state_in;
    uint16_t *conv_state_out;
    _Float16 *qk;  // [B][T][Hk][2][128]
    int B, T, Hk, Cc, conv;
    float eps_l2;
};

constexpr int kPrepTok = 32;  // tokens per prep workgroup

// grid (ceil(T/32), Hk, B).  Thread = (segment of 4 tokens, q|k, 8 channels).
__global__ __launch_bounds__(kThreads) void qk_prep_kernel(PrepArgs a) {
    const int tid = threadIdx.x;
    const int kh = blockIdx.y, b = blockIdx.z;
    const int cg = tid & 15;
    const int m = (tid >> 4) & 1;  // 0 = q, 1 = k
    const int seg = tid >> 5;
    const int t0 = blockIdx.x * kPrepTok + seg * 4;
    const uint16_t *src = m ? a.k : a.q;
    const int c = m * a.Hk * kD + kh * kD + cg * 8;  // conv channel of element 0

    float x[7][8];
#pragma unroll
    for (int rr = 0; rr < 7; ++rr) {
        const int t = t0 - 3 + rr;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (t >= 0 && t < a.T)
            raw = *reinterpret_cast<const uint4 *>(src + (((size_t)b * a.T + t) * a.Hk + kh) * kD + cg * 8);
        else if (t < 0 && a.conv && a.conv_state_in)
            raw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + (3 + t)) * a.Cc + c);
        unpack_bf16x8(raw, x[rr]);
    }
    float w[8][4];
    if (a.conv) {
        const uint4 *wp = reinterpret_cast<const uint4 *>(a.conv_w + (size_t)c * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float tmp[8];
            unpack_bf16x8(wp[i], tmp);
#pragma unroll
            for (int e = 0; e < 8; ++e) w[(8 * i + e) >> 2][(8 * i + e) & 3] = tmp[e];
        }
    }
    const float qscale = m ? 1.0f : 0.08838834764831845f;  // 1/sqrt(128) on q
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float u[8];
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (a.conv) {
                const float acc = w[e][0] * x[i][e] + w[e][1] * x[i + 1][e] + w[e][2] * x[i + 2][e] +
                                  w[e][3] * x[i + 3][e];
                u[e] = silu(acc);
            } else {
                u[e] = x[i + 3][e];
            }
            ss += u[e] * u[e];
        }
        ss = group_sum<16>(ss);
        const float sc = qscale / sqrtf(ss + a.eps_l2);
        const int t = t0 + i;
        if (t < a.T) {
            half8 hv;
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = static_cast<_Float16>(u[e] * sc);
            *reinterpret_cast<half8 *>(a.qk + ((((size_t)b * a.T + t) * a.Hk + kh) * 2 + m) * kD + cg * 8) = hv;
        }
    }

    // raw q/k inputs of the last three tokens -> conv state out
    if (blockIdx.x == 0 && a.conv && a.conv_state_out && tid < 96) {
        const int s = tid >> 5, mm = (tid >> 4) & 1;
        const int tau = a.T - 3 + s;
        const int cc = mm * a.Hk * kD + kh * kD + cg * 8;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (tau >= 0)
            raw = *reinterpret_cast<const uint4 *>((mm ? a.k : a.q) + (((size_t)b * a.T + tau) * a.Hk + kh) * kD + cg * 8);
        else if (a.conv_state_in)
            raw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + (3 + tau)) * a.Cc + cc);
        *reinterpret_cast<uint4 *>(a.conv_state_out + ((size_t)b * 3 + s) * a.Cc + cc) = raw;
    }
}

// ------------------------------------------------------------------------
// chain kernel
// ------------------------------------------------------------------------

struct ChainArgs {
    const _Float16 *qk;
    const uint16_t *v, *z, *conv_w, *norm_w, *conv_state_in;
    const float *g, *beta, *state_in;
    uint16_t *o, *conv_state_out;
    float *state_out;
    unsigned long long *mbox;  // [B*Hv][nslice][kRing][64]
    unsigned int *counters;    // [B*Hv]
    unsigned int *err;
    int B, T, Hk, Hv, r, Cc, conv, norm, n_items, grid;
    float eps_norm;
};

template <int BV>
struct Lds {
    static constexpr int NTJ = BV / 16;
    // byte offsets
    static constexpr size_t sQ = 0;                                    // fp16 [64][P128]   q^
    static constexpr size_t sK = sQ + 2 * kC * P128;                   // fp16 [64][P128]   k^
    static constexpr size_t sKT = sK + 2 * kC * P128;                  // fp16 [128][P64]   k^ transposed
    static constexpr size_t sV = sKT + 2 * kD * P64;                   // fp32 [64][BV+4]   conv(v) slice
    static constexpr size_t sL = sV + 4 * kC * (BV + 4);               // fp32 [64][PL]     strictly lower A
    static constexpr size_t sTd = sL + 4 * kC * PL;                    // fp32 [4][16][PTD] diagonal blocks of T
    static constexpr size_t sXT = sL;                                  // fp16 [BV][P64]    X^T   (aliases sL/sTd)
    static constexpr size_t sDT = sXT + 2 * BV * P64;                  // fp16 [BV][P64]    Delta^T (aliases)
    static constexpr size_t sT16T = sTd + 4 * 4 * 16 * PTD;            // fp16 [64][P64]    T transposed
    static constexpr size_t sTb = sT16T + 2 * kC * P64;                // fp16 [64][P64]    T diag(beta)
    static constexpr size_t sP = sTb + 2 * kC * P64;                   // fp16 [64][P64]    (Q K^T) o R
    static constexpr size_t sST = sP + 2 * kC * P64;                   // fp16 [BV][P128]   S^T slice
    static constexpr size_t sDTs = sST + 2 * BV * P128;                // fp16 [BV][P64]    (diag(e^{GC-G}) Delta)^T
    static constexpr size_t sVec = sDTs + 2 * BV * P64;                // fp32 [4][64]: G, beta, e^G, e^{GC-G}
    static constexpr size_t bytes = sVec + 4 * 4 * kC;
    static_assert(sDT + 2 * BV * P64 <= sT16T, "X/Delta alias overflows the L/Td region");
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Wait until the tagged word at p carries `tag`.  The wait is bounded: on a
// timeout the error word is raised and this thread stops waiting for the rest
// of the launch (`broken`), so a lost sibling cannot stall every later chunk.
__device__ __forceinline__ unsigned long long spin_load(unsigned long long *p, uint32_t tag, unsigned int *err,
                                                        int &broken) {
    unsigned long long w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t n = 0;
    while ((uint32_t)(w >> 32) != tag) {
        if (broken || ++n > kSpinLimit) {
            if (!broken) atomicOr(err, 1u);
            broken = 1;
            return 0ull;
        }
        __builtin_amdgcn_s_sleep(1);
        w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return w;
}

template <int BV>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs a) {
    using L = Lds<BV>;
    constexpr int NTJ = L::NTJ;
    constexpr int NSL = kD / BV;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    _Float16 *sQ = reinterpret_cast<_Float16 *>(smem + L::sQ);
    _Float16 *sK = reinterpret_cast<_Float16 *>(smem + L::sK);
    _Float16 *sKT = reinterpret_cast<_Float16 *>(smem + L::sKT);
    float *sV = reinterpret_cast<float *>(smem + L::sV);
    float *sL = reinterpret_cast<float *>(smem + L::sL);
    float *sTd = reinterpret_cast<float *>(smem + L::sTd);
    _Float16 *sXT = reinterpret_cast<_Float16 *>(smem + L::sXT);
    _Float16 *sDT = reinterpret_cast<_Float16 *>(smem + L::sDT);
    _Float16 *sT16T = reinterpret_cast<_Float16 *>(smem + L::sT16T);
    _Float16 *sTb = reinterpret_cast<_Float16 *>(smem + L::sTb);
    _Float16 *sP = reinterpret_cast<_Float16 *>(smem + L::sP);
    _Float16 *sST = reinterpret_cast<_Float16 *>(smem + L::sST);
    _Float16 *sDTs = reinterpret_cast<_Float16 *>(smem + L::sDTs);
    float *sG = reinterpret_cast<float *>(smem + L::sVec);
    float *sB = sG + kC;
    float *sEG = sB + kC;
    float *sEGC = sEG + kC;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, lq = lane >> 4;  // MFMA row/col within a tile, k-group

    // Blocks of sP and sTb above the diagonal are read as zeros by the
    // triangular products and never written: clear them once.
    for (int i = tid; i < kC * P64; i += kThreads) {
        const int row = i / P64, col = i % P64;
        if ((col >> 4) > (row >> 4)) {
            sP[i] = static_cast<_Float16>(0.0f);
            sTb[i] = static_cast<_Float16>(0.0f);
        }
    }

    // physical workgroup -> logical slot, so that consecutive slots share an XCD
    const int p = blockIdx.x;
    const int slot = (a.grid % 8 == 0) ? (p % 8) * (a.grid / 8) + p / 8 : p;
    const int nchunks = (a.T + kC - 1) / kC;
    float nw[NTJ];  // gated-norm weight of this lane's columns
    int broken = 0;  // set once a bounded wait has timed out

    for (int item = slot; item < a.n_items; item += a.grid) {
        const int chain = item / NSL, s = item % NSL;
        const int b = chain / a.Hv, h = chain % a.Hv, kh = h / a.r;
        const int sv0 = s * BV;
#pragma unroll
        for (int tj = 0; tj < NTJ; ++tj)
            nw[tj] = a.norm ? bf16_to_f32(a.norm_w[sv0 + 16 * tj + l16]) : 1.0f;

        // ---- state slice into accumulators: wave owns key-row tiles 2w, 2w+1
        floatx4 S[2][NTJ];
        {
            const float *src = a.state_in ? a.state_in + (size_t)chain * kD * kD : nullptr;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int tj = 0; tj < NTJ; ++tj)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * (2 * wave + u) + 4 * lq + e, j = sv0 + 16 * tj + l16;
                        S[u][tj][e] = src ? src[(size_t)i * kD + j] : 0.0f;
                    }
        }
        // fp16 copy of the state slice for the chunk's contractions
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int tj = 0; tj < NTJ; ++tj) {
                half4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = static_cast<_Float16>(S[u][tj][e]);
                *reinterpret_cast<half4 *>(sST + (16 * tj + l16) * P128 + 16 * (2 * wave + u) + 4 * lq) = hv;
            }

        floatx4 Oprev[NTJ];
        int have_prev = 0;

        for (int c = 0; c <= nchunks; ++c) {
            const bool compute = c < nchunks;
            const int t0 = c * kC;
            const int n = compute ? min(kC, a.T - t0) : 0;
            floatx4 Ocur[NTJ];

            if (compute) {
                // ================= A. loads and preprocessing
                for (int u = 0; u < 8; ++u) {
                    const int idx = tid + kThreads * u;
                    const int row = idx >> 5, part = (idx >> 4) & 1, cg = idx & 15;
                    half8 hv;
                    if (row < n) {
                        hv = *reinterpret_cast<const half8 *>(
                            a.qk + ((((size_t)b * a.T + t0 + row) * a.Hk + kh) * 2 + part) * kD + cg * 8);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) hv[e] = static_cast<_Float16>(0.0f);
                    }
                    _Float16 *dst = part ? sK : sQ;
                    *reinterpret_cast<half8 *>(dst + row * P128 + cg * 8) = hv;
                    if (part) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) sKT[(cg * 8 + e) * P64 + row] = hv[e];
                    }
                }
                if (wave == 0) {
                    const bool valid = lane < n;
                    const size_t gi = ((size_t)b * a.T + t0 + lane) * a.Hv + h;
                    float gv = valid ? a.g[gi] : 0.0f;
                    const float bv = valid ? a.beta[gi] : 0.0f;
                    // inclusive prefix sum over the chunk
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) {
                        const float t = __shfl_up(gv, o, 64);
                        if (lane >= o) gv += t;
                    }
                    const float gc = __shfl(gv, 63, 64);
                    sG[lane] = gv;
                    sB[lane] = bv;
                    sEG[lane] = __expf(gv);
                    sEGC[lane] = __expf(gc - gv);
                }
                {
                    constexpr int NCG = BV / 8;
                    constexpr int RSTEP = kThreads / NCG;
                    const int cg = tid % NCG;
                    const int ch = 2 * a.Hk * kD + h * kD + sv0 + cg * 8;  // conv channel
                    float w[8][4];
                    if (a.conv) {
                        const uint4 *wp = reinterpret_cast<const uint4 *>(a.conv_w + (size_t)ch * 4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float tmp[8];
                            unpack_bf16x8(wp[i], tmp);
#pragma unroll
                            for (int e = 0; e < 8; ++e) w[(8 * i + e) >> 2][(8 * i + e) & 3] = tmp[e];
                        }
                    }
                    for (int row = tid / NCG; row < kC; row += RSTEP) {
                        float u[8];
                        if (row < n) {
                            float x[4][8];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int tau = t0 + row - 3 + j;
                                uint4 raw = make_uint4(0, 0, 0, 0);
                                if (j == 3 || a.conv) {
                                    if (tau >= 0)
                                        raw = *reinterpret_cast<const uint4 *>(
                                            a.v + (((size_t)b * a.T + tau) * a.Hv + h) * kD + sv0 + cg * 8);
                                    else if (a.conv_state_in)
                                        raw = *reinterpret_cast<const uint4 *>(
                                            a.conv_state_in + ((size_t)b * 3 + (3 + tau)) * a.Cc + ch);
                                }
                                unpack_bf16x8(raw, x[j]);
                            }
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                u[e] = a.conv ? silu(w[e][0] * x[0][e] + w[e][1] * x[1][e] + w[e][2] * x[2][e] +
                                                     w[e][3] * x[3][e])
                                              : x[3][e];
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) u[e] = 0.0f;
                        }
                        float4 *dst = reinterpret_cast<float4 *>(sV + row * (BV + 4) + cg * 8);
                        dst[0] = make_float4(u[0], u[1], u[2], u[3]);
                        dst[1] = make_float4(u[4], u[5], u[6], u[7]);
                    }
                }
                __syncthreads();

                // ================= B1. K K^T -> L (fp32), Q K^T o R -> P (fp16)
                for (int task = wave; task < 20; task += 4) {
                    const bool isP = task >= 10;
                    const int tt = isP ? task - 10 : task;
                    const int ti = tt < 1 ? 0 : tt < 3 ? 1 : tt < 6 ? 2 : 3;
                    const int tj = tt - ti * (ti + 1) / 2;
                    const _Float16 *Aop = isP ? sQ : sK;
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const half8 av = lds_half8(Aop + (16 * ti + l16) * P128 + 32 * ks + 8 * lq);
                        const half8 bv = lds_half8(sK + (16 * tj + l16) * P128 + 32 * ks + 8 * lq);
                        acc = mfma16x16x32(av, bv, acc);
                    }
                    const int col = 16 * tj + l16;
                    const float gcol = sG[col];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 16 * ti + 4 * lq + e;
                        const float rdec = __expf(sG[row] - gcol);
                        if (isP) {
                            sP[row * P64 + col] = static_cast<_Float16>(col <= row ? acc[e] * rdec : 0.0f);
                        } else {
                            sL[row * PL + col] = col < row ? sB[row] * acc[e] * rdec : 0.0f;
                        }
                    }
                }
                __syncthreads();

                // ================= B2. diagonal 16x16 blocks of T = (I + L)^{-1}
                if (lane < 16) {
                    const int w0 = 16 * wave, cidx = lane;
                    float x[16];
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        float acc = 0.0f;
#pragma unroll
                        for (int mm = 0; mm < rr; ++mm) acc += sL[(w0 + rr) * PL + w0 + mm] * x[mm];
                        x[rr] = (rr == cidx) ? 1.0f : (rr < cidx ? 0.0f : -acc);
                    }
                    const float bc = sB[w0 + cidx];
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        sTd[(wave * 16 + rr) * PTD + cidx] = x[rr];
                        sT16T[(w0 + cidx) * P64 + w0 + rr] = static_cast<_Float16>(x[rr]);
                        sTb[(w0 + rr) * P64 + w0 + cidx] = static_cast<_Float16>(x[rr] * bc);
                    }
                }
                __syncthreads();

                // ================= B3. off-diagonal blocks, column block J = wave:
                //   T_IJ = -T_II * sum_{K=J}^{I-1} L_IK T_KJ
                if (wave < 3) {
                    const int J = wave;
                    const float bcol = sB[16 * J + l16];
                    for (int I = J + 1; I < 4; ++I) {
                        floatx4 y = {0.f, 0.f, 0.f, 0.f};
                        for (int K = J; K < I; ++K) {
                            half4 av, bv;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                av[e] = static_cast<_Float16>(sL[(16 * I + l16) * PL + 16 * K + 4 * lq + e]);
                            bv = lds_half4(sT16T + (16 * J + l16) * P64 + 16 * K + 4 * lq);
                            y = mfma16x16x16(av, bv, y);
                        }
                        // y's accumulator layout is the B-operand layout of the next product
                        half4 yb, tv;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            yb[e] = static_cast<_Float16>(y[e]);
                            tv[e] = static_cast<_Float16>(sTd[(I * 16 + l16) * PTD + 4 * lq + e]);
                        }
                        floatx4 t = {0.f, 0.f, 0.f, 0.f};
                        t = mfma16x16x16(tv, yb, t);
                        half4 th;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            th[e] = static_cast<_Float16>(-t[e]);
                            sTb[(16 * I + 4 * lq + e) * P64 + 16 * J + l16] = static_cast<_Float16>(-t[e] * bcol);
                        }
                        *reinterpret_cast<half4 *>(sT16T + (16 * J + l16) * P64 + 16 * I + 4 * lq) = th;
                        wave_lds_sync();
                    }
                }
                __syncthreads();

                // ================= C1. K S and Q S (token-row tile = wave)
                floatx4 ks_acc[NTJ];
                {
                    half8 ak[4], aq[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        ak[ks] = lds_half8(sK + (16 * wave + l16) * P128 + 32 * ks + 8 * lq);
                        aq[ks] = lds_half8(sQ + (16 * wave + l16) * P128 + 32 * ks + 8 * lq);
                    }
#pragma unroll
                    for (int tj = 0; tj < NTJ; ++tj) {
                        floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) {
                            const half8 bv = lds_half8(sST + (16 * tj + l16) * P128 + 32 * ks + 8 * lq);
                            a1 = mfma16x16x32(ak[ks], bv, a1);
                            a2 = mfma16x16x32(aq[ks], bv, a2);
                        }
                        ks_acc[tj] = a1;
                        Ocur[tj] = a2;
                    }
                }
#pragma unroll
                for (int tj = 0; tj < NTJ; ++tj) {
                    half4 xh;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 16 * wave + 4 * lq + e, col = 16 * tj + l16;
                        const float eg = sEG[row];
                        xh[e] = static_cast<_Float16>(sV[row * (BV + 4) + col] - eg * ks_acc[tj][e]);
                        Ocur[tj][e] *= eg;
                    }
                    *reinterpret_cast<half4 *>(sXT + (16 * tj + l16) * P64 + 16 * wave + 4 * lq) = xh;
                }
                __syncthreads();

                // ================= C2. Delta = T diag(beta) X  (row tile = wave, triangular)
                {
                    const int nks = wave < 2 ? 1 : 2;
#pragma unroll
                    for (int tj = 0; tj < NTJ; ++tj) {
                        floatx4 dacc = {0.f, 0.f, 0.f, 0.f};
                        for (int ks = 0; ks < nks; ++ks) {
                            const half8 av = lds_half8(sTb + (16 * wave + l16) * P64 + 32 * ks + 8 * lq);
                            const half8 bv = lds_half8(sXT + (16 * tj + l16) * P64 + 32 * ks + 8 * lq);
                            dacc = mfma16x16x32(av, bv, dacc);
                        }
                        half4 dh, dsh;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int row = 16 * wave + 4 * lq + e;
                            dh[e] = static_cast<_Float16>(dacc[e]);
                            dsh[e] = static_cast<_Float16>(dacc[e] * sEGC[row]);
                        }
                        *reinterpret_cast<half4 *>(sDT + (16 * tj + l16) * P64 + 16 * wave + 4 * lq) = dh;
                        *reinterpret_cast<half4 *>(sDTs + (16 * tj + l16) * P64 + 16 * wave + 4 * lq) = dsh;
                    }
                }
                __syncthreads();

                // ================= C3. O += P Delta;  S = e^{G_C} S + K^T Delta~
                {
                    const int nks = wave < 2 ? 1 : 2;
#pragma unroll
                    for (int tj = 0; tj < NTJ; ++tj)
                        for (int ks = 0; ks < nks; ++ks) {
                            const half8 av = lds_half8(sP + (16 * wave + l16) * P64 + 32 * ks + 8 * lq);
                            const half8 bv = lds_half8(sDT + (16 * tj + l16) * P64 + 32 * ks + 8 * lq);
                            Ocur[tj] = mfma16x16x32(av, bv, Ocur[tj]);
                        }
                    const float dC = sEG[kC - 1];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int ti = 2 * wave + u;
                        half8 av[2];
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) av[ks] = lds_half8(sKT + (16 * ti + l16) * P64 + 32 * ks + 8 * lq);
#pragma unroll
                        for (int tj = 0; tj < NTJ; ++tj) {
                            floatx4 acc = S[u][tj] * dC;
#pragma unroll
                            for (int ks = 0; ks < 2; ++ks) {
                                const half8 bv = lds_half8(sDTs + (16 * tj + l16) * P64 + 32 * ks + 8 * lq);
                                acc = mfma16x16x32(av[ks], bv, acc);
                            }
                            S[u][tj] = acc;
                            half4 hv;
#pragma unroll
                            for (int e = 0; e < 4; ++e) hv[e] = static_cast<_Float16>(acc[e]);
                            *reinterpret_cast<half4 *>(sST + (16 * tj + l16) * P128 + 16 * ti + 4 * lq) = hv;
                        }
                    }
                }

                // per-row partial sums of squares over this slice's columns -> mailbox
                if (a.norm && NSL > 1) {
                    float ssr[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float acc = 0.0f;
#pragma unroll
                        for (int tj = 0; tj < NTJ; ++tj) acc += Ocur[tj][e] * Ocur[tj][e];
                        ssr[e] = group_sum<16>(acc);
                    }
                    if (l16 == 0) {
                        unsigned long long *mb =
                            a.mbox + (((size_t)chain * NSL + s) * kRing + (c % kRing)) * kC + 16 * wave + 4 * lq;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const unsigned long long wv =
                                ((unsigned long long)(uint32_t)(c + 1) << 32) | __float_as_uint(ssr[e]);
                            __hip_atomic_store(mb + e, wv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                }
            }

            // ================= D. gated norm + store of one chunk's rows
            // With sibling slices the chunk finished one iteration ago is
            // written (its partial sums had a full chunk to arrive).
            const bool deferred = a.norm && NSL > 1;
            const int oc = deferred ? c - 1 : c;
            if ((deferred && have_prev) || (!deferred && compute)) {
                floatx4 *Ob = deferred ? Oprev : Ocur;
                const int ot0 = oc * kC;
                float rstd[4] = {1.f, 1.f, 1.f, 1.f};
                if (a.norm) {
                    float tot;
                    if (NSL > 1) {
                        tot = 0.0f;
                        for (int sib = lq; sib < NSL; sib += 4) {
                            unsigned long long *mb =
                                a.mbox + (((size_t)chain * NSL + sib) * kRing + (oc % kRing)) * kC + 16 * wave + l16;
                            const unsigned long long wv = spin_load(mb, (uint32_t)(oc + 1), a.err, broken);
                            tot += __uint_as_float((uint32_t)wv);
                        }
                        tot += __shfl_xor(tot, 16, 64);
                        tot += __shfl_xor(tot, 32, 64);
                    } else {
                        float acc[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float t = 0.0f;
#pragma unroll
                            for (int tj = 0; tj < NTJ; ++tj) t += Ob[tj][e] * Ob[tj][e];
                            acc[e] = group_sum<16>(t);
                        }
                        // lane (row % 16) collects its row's total
                        tot = 0.0f;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v0 = __shfl(acc[e], (l16 >> 2) * 16, 64);
                            if ((l16 & 3) == e) tot = v0;
                        }
                    }
                    const float rs = 1.0f / sqrtf(tot * (1.0f / kD) + a.eps_norm);
#pragma unroll
                    for (int e = 0; e < 4; ++e) rstd[e] = __shfl(rs, 4 * lq + e, 64);
                }
#pragma unroll
                for (int tj = 0; tj < NTJ; ++tj)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 16 * wave + 4 * lq + e;
                        const int t = ot0 + row;
                        if (t < a.T) {
                            const size_t off = (((size_t)b * a.T + t) * a.Hv + h) * kD + sv0 + 16 * tj + l16;
                            float y = Ob[tj][e];
                            if (a.norm) y = nw[tj] * (y * rstd[e]) * silu(bf16_to_f32(a.z[off]));
                            a.o[off] = f32_to_bf16(y);
                        }
                    }
            }
            if (compute) {
#pragma unroll
                for (int tj = 0; tj < NTJ; ++tj) Oprev[tj] = Ocur[tj];
                have_prev = 1;
            }
            __syncthreads();
        }

        // ---- final state slice
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int tj = 0; tj < NTJ; ++tj)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * (2 * wave + u) + 4 * lq + e, j = sv0 + 16 * tj + l16;
                    a.state_out[(size_t)chain * kD * kD + (size_t)i * kD + j] = S[u][tj][e];
                }
        // ---- raw v inputs of the last three tokens -> conv state out
        if (a.conv && a.conv_state_out && tid < 3 * (BV / 8)) {
            const int sidx = tid / (BV / 8), cg = tid % (BV / 8);
            const int tau = a.T - 3 + sidx;
            const int ch = 2 * a.Hk * kD + h * kD + sv0 + cg * 8;
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (tau >= 0)
                raw = *reinterpret_cast<const uint4 *>(a.v + (((size_t)b * a.T + tau) * a.Hv + h) * kD + sv0 + cg * 8);
            else if (a.conv_state_in)
                raw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + (3 + tau)) * a.Cc + ch);
            *reinterpret_cast<uint4 *>(a.conv_state_out + ((size_t)b * 3 + sidx) * a.Cc + ch) = raw;
        }
        // ---- the last slice of a chain to finish clears the chain's mailbox
        if (a.norm && NSL > 1) {
            __syncthreads();
            __shared__ unsigned int last;
            if (tid == 0) {
                const unsigned int old =
                    __hip_atomic_fetch_add(a.counters + chain, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                last = (old == NSL - 1) ? 1u : 0u;
            }
            __syncthreads();
            if (last) {
                unsigned long long *mb = a.mbox + (size_t)chain * NSL * kRing * kC;
                for (int i = tid; i < NSL * kRing * kC; i += kThreads)
                    __hip_atomic_store(mb + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (tid == 0) __hip_atomic_store(a.counters + chain, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int BV>
int launch_chain(const ChainArgs &base, hipStream_t stream) {
    ChainArgs a = base;
    constexpr size_t lds = Lds<BV>::bytes;
    auto fn = chain_kernel<BV>;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
        return -1;
    int dev = 0, ncu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(fn), kThreads, lds) !=
            hipSuccess ||
        per_cu < 1)
        return -1;
    constexpr int NSL = kD / BV;
    const int cap = ncu * per_cu;
    const int unit = 8 * NSL;  // keeps sibling slices contiguous inside one XCD's share
    int grid = a.n_items <= cap ? ((a.n_items + unit - 1) / unit) * unit : (cap / unit) * unit;
    if (grid > cap) grid = (cap / unit) * unit;
    if (grid < unit) grid = unit <= cap ? unit : cap - cap % NSL;
    if (grid < NSL) return -1;
    a.grid = grid;
    void *args[] = {&a};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(fn), dim3(grid), dim3(kThreads),
                                                    args, (unsigned)lds, stream);
    return e == hipSuccess ? 0 : -1;
}

} // namespace

int plan_prefill(int B, int T, int Hk, int Hv, PrefillPlan *plan) {
    const long long chains = (long long)B * Hv;
    int nsl = 2;
    while (nsl < 8 && chains * nsl * 2 <= kCUs) nsl *= 2;
    plan->nslice = nsl;
    plan->bv = kD / nsl;
    plan->qk_bytes = align256((size_t)B * T * Hk * 2 * kD * sizeof(_Float16));
    plan->mbox_bytes = align256((size_t)chains * nsl * kRing * kC * sizeof(unsigned long long)) +
                       align256((size_t)chains * sizeof(unsigned int)) + 256;
    return 0;
}

int launch_prefill(const PrefillParams &p, const PrefillPlan &plan, hipStream_t stream) {
    unsigned char *ws = static_cast<unsigned char *>(p.workspace);
    _Float16 *qk = reinterpret_cast<_Float16 *>(ws);
    unsigned char *mb = ws + plan.qk_bytes;
    const size_t chains = (size_t)p.B * p.Hv;
    const size_t mbox_words = align256(chains * plan.nslice * kRing * kC * sizeof(unsigned long long));
    unsigned int *counters = reinterpret_cast<unsigned int *>(mb + mbox_words);
    unsigned int *err = reinterpret_cast<unsigned int *>(mb + mbox_words + align256(chains * sizeof(unsigned int)));

    PrepArgs pa;
    pa.q = p.q; pa.k = p.k; pa.conv_w = p.conv_w; pa.conv_state_in = p.conv_state_in;
    pa.conv_state_out = p.conv_state_out; pa.qk = qk;
    pa.B = p.B; pa.T = p.T; pa.Hk = p.Hk; pa.Cc = 2 * p.Hk * kD + p.Hv * kD;
    pa.conv = p.conv_width == 4; pa.eps_l2 = p.eps_l2;
    const dim3 pgrid((unsigned)((p.T + kPrepTok - 1) / kPrepTok), (unsigned)p.Hk, (unsigned)p.B);
    hipLaunchKernelGGL(qk_prep_kernel, pgrid, dim3(kThreads), 0, stream, pa);
    if (hipGetLastError() != hipSuccess) return -1;

    ChainArgs a;
    a.qk = qk; a.v = p.v; a.z = p.z; a.conv_w = p.conv_w; a.norm_w = p.norm_w; a.conv_state_in = p.conv_state_in;
    a.g = p.g; a.beta = p.beta; a.state_in = p.state_in;
    a.o = p.o; a.conv_state_out = p.conv_state_out; a.state_out = p.state_out;
    a.mbox = reinterpret_cast<unsigned long long *>(mb); a.counters = counters; a.err = err;
    a.B = p.B; a.T = p.T; a.Hk = p.Hk; a.Hv = p.Hv; a.r = p.Hv / p.Hk;
    a.Cc = pa.Cc; a.conv = pa.conv; a.norm = p.norm;
    a.n_items = (int)(chains * plan.nslice); a.grid = 0;
    a.eps_norm = p.eps_norm;
    switch (plan.bv) {
    case 16: return launch_chain<16>(a, stream);
    case 32: return launch_chain<32>(a, stream);
    case 64: return launch_chain<64>(a, stream);
    default: return -1;
    }
}

} // namespace gdn
