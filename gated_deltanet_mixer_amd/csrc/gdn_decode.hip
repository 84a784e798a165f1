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
// value heads; for each, 512 threads hold the 128x128 state in registers
// (thread = 4 value columns x 8 key rows, float4 loads: a wave reads two
// consecutive 512-byte rows per instruction), reduce S^T k and S^T q in one
// pass, and write S' = a S + k d^T.
//
// Memory schedule: the step moves 128 KiB of state per value head and little
// else, so the kernel keeps state traffic in flight at all times.  Every small
// input of the workgroup (raw q/k/v, conv window and weights, z, g, beta) is
// requested first, then the first head's state, and only then does the conv
// run; each head requests the next head's state before it starts on its own.
// Barriers order LDS only, so stores and prefetches stay in flight across
// them, and z waits in LDS: on this target one counter tracks loads and
// stores, so a global load issued after the state stores would wait for them.
//
// Read-out identity: with S' = a S + k d^T, o = S'^T q = a (S^T q) + (q.k) d,
// so both reductions come from the single read of S.  This follows from the
// decay -> predict -> correct -> read order of "How Qwen3.5 works" §9.6.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kD = 128;
constexpr int kRows = kD / (kThreads / 32);  // state rows per thread (8)

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

// Buffer resource over `bytes` bytes from p: the state tiles are addressed as one
// per-thread offset plus a wave-uniform offset per row block and head, so the eight
// loads or stores of a tile share one address register.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf(const void *p, unsigned int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}
// Cache policy of the state traffic, which every call streams once: loads marked
// non-temporal (nt) and stores written through at agent scope (sc1).  Measured on a
// read-modify-write of 805 MB in 64 KiB pieces, the decode's pattern: 6.05 TB/s
// against 5.45 TB/s with the default policy.  Only the caching changes; the kernel
// boundary orders the stores for whatever reads the state next.
constexpr int kStateLoadPolicy = 2;    // nt
constexpr int kStateStorePolicy = 16;  // sc1

// LDS of one workgroup, in floats, for T tokens and r value heads per key head.
struct DecodeLds {
    int nu, U, Qn, Kn, Red, D, Z, Al, Be, QK, Misc, total;
    __host__ __device__ DecodeLds(int T, int r) {
        nu = 2 * kD + kD * r;            // conv outputs of one token: q, k, then the r heads' v
        U = 0;                           // [T][nu]
        Qn = U + T * nu;                 // [T][128] normalised q (incl. 1/sqrt(128))
        Kn = Qn + T * kD;                // [T][128] normalised k
        Red = Kn + T * kD;               // [kWaves][2][128] partial column sums
        D = Red + kWaves * 2 * kD;       // [128] correction d
        Z = D + kD;                      // [r][T][128] z as bf16 (half a float each)
        Al = Z + (r * T * kD) / 2;       // [r][T] e^g
        Be = Al + r * T;                 // [r][T] beta
        QK = Be + r * T;                 // [kMaxTokens] q^.k^
        Misc = QK + kMaxTokens;          // [2] norm partials
        total = Misc + 2;
    }
};

// The thread's conv item: 8 channels of q (it < 16), k (16 <= it < 32) or the v of
// value head (it - 32) / 16.  Sets the first raw input, the stride from one token's
// row to the next and the conv channel of element 0.
__device__ __forceinline__ void conv_item(const DecodeArgs &a, int b, int kh, int it, const uint16_t *&xp,
                                          size_t &xstride, int &c) {
    const int T = a.T;
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
        const int h = kh * a.r + hr;
        c = 2 * a.Hk * kD + h * kD + j8 * 8;
        xp = a.v + ((size_t)b * T * a.Hv + h) * kD + j8 * 8;
        xstride = (size_t)a.Hv * kD;
    }
}

// Raw inputs of one conv item in time order: the three stored ones, then the T new
// tokens; and the item's conv weights.
template <int MAXT>
struct ConvRaw {
    uint4 raw[3 + MAXT];
    uint4 w[4];
};

template <int MAXT>
__device__ __forceinline__ void conv_load(const DecodeArgs &a, int b, int kh, int it, int T, ConvRaw<MAXT> &cr) {
    const uint16_t *xp;
    size_t xstride;
    int c;
    conv_item(a, b, kh, it, xp, xstride, c);
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
        if (t < T) cr.raw[3 + t] = *reinterpret_cast<const uint4 *>(xp + t * xstride);
    if (a.conv) {
        const uint16_t *cs = a.conv_state + (size_t)b * 3 * a.Cc + c;
#pragma unroll
        for (int s = 0; s < 3; ++s) cr.raw[s] = *reinterpret_cast<const uint4 *>(cs + s * a.Cc);
        const uint4 *wp = reinterpret_cast<const uint4 *>(a.conv_w + (size_t)c * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) cr.w[i] = wp[i];
    }
}

// Conv + SiLU of one item for every token -> sU; the window after each token goes to
// its snapshot, the one after the last token back in place.
template <int MAXT>
__device__ __forceinline__ void conv_run(const DecodeArgs &a, int b, int kh, int it, int T, int nu, float *sU,
                                         const ConvRaw<MAXT> &cr) {
    const uint16_t *xp;
    size_t xstride;
    int c;
    conv_item(a, b, kh, it, xp, xstride, c);
    if (a.conv) {
        uint16_t *cs = a.conv_state + (size_t)b * 3 * a.Cc + c;
        // weights and inputs stay packed (two bf16 per word) and are widened one channel
        // at a time, which keeps the registers free for the state in flight
        auto half_of = [](const uint4 &v, int e) {
            const uint32_t wd = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
            return (e & 1) ? __uint_as_float(wd & 0xffff0000u) : __uint_as_float(wd << 16);
        };
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            if (t < T) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // taps of channel e: conv_w[c + e][0..3], in word (e / 2) of cr.w
                    const uint4 &wv = cr.w[e >> 1];
                    const int o = 4 * (e & 1);
                    // tap 3 multiplies the current token, tap 0 the one three before it
                    const float acc = half_of(wv, o + 0) * half_of(cr.raw[t], e) +
                                      half_of(wv, o + 1) * half_of(cr.raw[t + 1], e) +
                                      half_of(wv, o + 2) * half_of(cr.raw[t + 2], e) +
                                      half_of(wv, o + 3) * half_of(cr.raw[t + 3], e);
                    sU[t * nu + it * 8 + e] = silu(acc);
                }
                // the window after token t: raw[t+1 .. t+3]; the last one replaces the stored window
                uint16_t *dst = t == T - 1 ? cs
                                : a.conv_snaps ? a.conv_snaps + ((size_t)t * a.B + b) * 3 * a.Cc + c
                                               : nullptr;
                if (dst) {
#pragma unroll
                    for (int s = 0; s < 3; ++s) *reinterpret_cast<uint4 *>(dst + s * a.Cc) = cr.raw[t + 1 + s];
                }
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            if (t < T) {
                float x[8];
                unpack_bf16x8(cr.raw[3 + t], x);
#pragma unroll
                for (int e = 0; e < 8; ++e) sU[t * nu + it * 8 + e] = x[e];
            }
        }
    }
}

// MAXT: the tokens per call the register arrays are sized for (1, 2, 4 or 8).  Up to 4
// tokens two workgroups share a CU; 8 tokens' raw rows need more registers than that leaves.
template <int MAXT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MAXT <= 4 ? 4 : 2))) void decode_kernel(DecodeArgs a) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int b = blockIdx.x / a.Hk;
    const int kh = blockIdx.x % a.Hk;
    const int r = a.r, T = MAXT == 1 ? 1 : a.T;
    constexpr bool kPF = MAXT == 1;  // the next head's state is prefetched
    const DecodeLds L(T, r);
    const int nu = L.nu;

    extern __shared__ float smem[];
    float *sU = smem + L.U, *sQn = smem + L.Qn, *sKn = smem + L.Kn, *sRed = smem + L.Red, *sD = smem + L.D;
    uint16_t *sZ = reinterpret_cast<uint16_t *>(smem + L.Z);
    float *sAl = smem + L.Al, *sBe = smem + L.Be, *sQK = smem + L.QK, *sMisc = smem + L.Misc;

    // thread tile of a head's state: columns 4 jg .. 4 jg + 3, rows rg + 16 m
    const int jg = tid & 31, rg = tid >> 5;
    // the item's r heads are consecutive: one resource covers them (r * 64 KiB)
    constexpr int kHeadBytes = kD * kD * 4;
    const __amdgpu_buffer_rsrc_t rstate = buf(a.state + ((size_t)b * a.Hv + kh * r) * kD * kD, r * kHeadBytes);
    const int toff = (rg * (kD / 4) + jg) * 16;  // the thread's float4 in row block 0
    // dummy: every lane reads the same eight 16-byte pieces of head hr (cached after the
    // first wave), so that a prefetch slot is always filled by the same number of loads
    auto load_state = [&](floatx4 (&S)[kRows], int hr, bool dummy) __attribute__((always_inline)) {
        const int vo = dummy ? 0 : toff;
#pragma unroll
        for (int m = 0; m < kRows; ++m)
            S[m] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rstate, vo, hr * kHeadBytes + m * 16 * kD * 4, kStateLoadPolicy));
    };

    // ---- 0. every small input first: the conv item's raw rows and weights, z, the gates
    const int n_items = nu / 8;
    ConvRaw<MAXT> cr;
    if (tid < n_items) conv_load<MAXT>(a, b, kh, tid, T, cr);
    const int nz = a.norm ? r * T * (kD / 8) : 0;  // 8 values of z per thread: [hr][t][j8]
    uint4 zr = make_uint4(0, 0, 0, 0);
    auto z_at = [&](int i) {
        const int hr = i / (T * 16), t = (i / 16) % T, j8 = i % 16;
        return reinterpret_cast<const uint4 *>(a.z + (((size_t)b * T + t) * a.Hv + kh * r + hr) * kD + j8 * 8);
    };
    if (tid < nz) zr = *z_at(tid);
    float g_raw = 0.0f, b_raw = 0.0f, alog = 0.0f, dtb = 0.0f;
    const int ngt = r * T;  // gates: [hr][t]
    if (tid < ngt) {
        const int hr = tid / T, t = tid % T;
        const size_t ht = ((size_t)b * T + t) * a.Hv + kh * r + hr;
        g_raw = a.g[ht];
        b_raw = a.beta[ht];
        if (a.A_log) {
            alog = a.A_log[kh * r + hr];
            dtb = a.dt_bias[kh * r + hr];
        }
    }
    // the norm weight, loaded by every thread from a valid address (q when there is no
    // norm) so that no branch makes the compiler wait for it before the state is requested
    const uint16_t nw_raw = (a.norm ? a.norm_w : a.q)[tid & (kD - 1)];
    __builtin_amdgcn_sched_barrier(0);
    // the first value head's state, in flight while the conv runs (with several tokens the
    // raw rows of all of them fill the registers: then it is requested after the conv)
    floatx4 S[kRows], Sn[kRows];
    if (kPF) load_state(Sn, 0, false);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 1. conv window shift + conv + SiLU on the owned channels, every token
    if (tid < n_items) conv_run<MAXT>(a, b, kh, tid, T, nu, sU, cr);
    for (int it = tid + kThreads; it < n_items; it += kThreads) {  // more than 30 value heads per key head
        ConvRaw<MAXT> cx;
        conv_load<MAXT>(a, b, kh, it, T, cx);
        conv_run<MAXT>(a, b, kh, it, T, nu, sU, cx);
    }
    if (tid < nz) *reinterpret_cast<uint4 *>(sZ + tid * 8) = zr;
    auto gate_item = [&](int i, float gl, float bt, float A_log, float dt_bias) {
        if (a.A_log) {  // gates from their logits
            gl = gate_g(gl, A_log, dt_bias);
            bt = gate_beta(bt);
        }
        sAl[i] = __expf(gl);
        sBe[i] = bt;
    };
    if (tid < ngt) gate_item(tid, g_raw, b_raw, alog, dtb);
    // more than 512 z pieces or gates (many value heads per key head): a second pass
    for (int i = tid + kThreads; i < nz; i += kThreads) *reinterpret_cast<uint4 *>(sZ + i * 8) = *z_at(i);
    for (int i = tid + kThreads; i < ngt; i += kThreads) {
        const int h = kh * r + i / T;
        const size_t ht = ((size_t)b * T + i % T) * a.Hv + h;
        gate_item(i, a.g[ht], a.beta[ht], a.A_log ? a.A_log[h] : 0.0f, a.A_log ? a.dt_bias[h] : 0.0f);
    }
    lds_barrier();

    // ---- 2. per token: L2 norms of q and k and the raw q.k (one wave per task)
    for (int task = wave; task < 3 * T; task += kWaves) {
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
    lds_barrier();

    // ---- 3. value heads: S in registers through the T tokens.
    // Two LDS barriers per token: the partial sums are read before the second, and the
    // next writes of sRed, sD and sMisc come after the next token's first, which no
    // thread reaches before it has used what it read.  Outputs wait in LDS (in the slot
    // of the z value they were gated with) and leave in one pass at the end.
    // One step (MAXT == 1): the next head's state is requested before the work on a head
    // starts, into Sn, and copied to S when the head is done; the last head fills the slot
    // with dummy loads, so that every head issues the same memory operations and S never
    // waits on a load.  Several tokens keep one state in registers (two would not fit
    // beside the tokens' conv rows): a head's state is requested as the head starts, and
    // T tokens of work and snapshot stores follow each request.
    const float nwj = (a.norm && tid < kD) ? bf16_to_f32(nw_raw) : 1.0f;
    if (kPF) {
        // The first head's state has had the conv and the norms to arrive.  An explicit
        // wait here also tells the compiler that nothing is pending on S when the head
        // loop starts (otherwise it keeps waiting on this load in every iteration).
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
#pragma unroll
        for (int m = 0; m < kRows; ++m) S[m] = Sn[m];
    }
    for (int hr = 0; hr < r; ++hr) {
        if (kPF)
            load_state(Sn, hr + 1 < r ? hr + 1 : hr, hr + 1 >= r);
        else
            load_state(S, hr, false);
        __builtin_amdgcn_sched_barrier(0);
        for (int t = 0; t < T; ++t) {
            const float *qn = sQn + t * kD, *kn = sKn + t * kD;
            float pk[4] = {0, 0, 0, 0}, pq[4] = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < kRows; ++m) {
                const float kv = kn[rg + 16 * m], qv = qn[rg + 16 * m];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pk[e] = __builtin_fmaf(S[m][e], kv, pk[e]);
                    pq[e] = __builtin_fmaf(S[m][e], qv, pq[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pk[e] += __shfl_xor(pk[e], 32, 64);
                pq[e] += __shfl_xor(pq[e], 32, 64);
            }
            if (lane < 32) {
                *reinterpret_cast<float4 *>(sRed + (wave * 2 + 0) * kD + 4 * jg) = make_float4(pk[0], pk[1], pk[2], pk[3]);
                *reinterpret_cast<float4 *>(sRed + (wave * 2 + 1) * kD + 4 * jg) = make_float4(pq[0], pq[1], pq[2], pq[3]);
            }
            lds_barrier();

            const float alpha = sAl[hr * T + t];
            float oj = 0.0f;
            if (tid < kD) {
                const int j = tid;
                float PK = 0.0f, PQ = 0.0f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    PK += sRed[(w * 2 + 0) * kD + j];
                    PQ += sRed[(w * 2 + 1) * kD + j];
                }
                const float vj = sU[t * nu + 2 * kD + hr * kD + j];
                // fused multiply-adds in a fixed order here and in the update below, so that every
                // instantiation (one step, several tokens) rounds alike
                const float d = sBe[hr * T + t] * __builtin_fmaf(-alpha, PK, vj);
                oj = __builtin_fmaf(sQK[t], d, alpha * PQ);
                sD[j] = d;
                if (a.norm) {
                    const float ss = wave_sum(oj * oj);
                    if (lane == 0) sMisc[wave] = ss;
                }
            }
            lds_barrier();

            // S' = a S + k d^T: in place after the last token, as a snapshot after the others
            const floatx4 d4 = reinterpret_cast<const floatx4 *>(sD)[jg];
            const bool keep = t == T - 1 || a.state_snaps;
            const __amdgpu_buffer_rsrc_t rdst =
                t == T - 1 || !a.state_snaps
                    ? rstate
                    : buf(a.state_snaps + (((size_t)t * a.B + b) * a.Hv + kh * r) * kD * kD, r * kHeadBytes);
#pragma unroll
            for (int m = 0; m < kRows; ++m) {
                const float kv = kn[rg + 16 * m];
                floatx4 sv = S[m];
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[e] = __builtin_fmaf(kv, d4[e], alpha * sv[e]);
                S[m] = sv;
                // The whole offset goes in the vector offset and the scalar offset is the constant
                // 0: the compiler then models the hazard of a VALU write to the data registers of
                // a wide store right behind it (it does not for a register scalar offset), and
                // inserts the wait state itself.
                if (keep)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sv), rdst,
                                                           toff + hr * kHeadBytes + m * 16 * kD * 4, 0,
                                                           kStateStorePolicy);
            }

            if (tid < kD) {
                const int j = tid;
                uint16_t *slot = sZ + (hr * T + t) * kD + j;
                float y = oj;
                if (a.norm) {
                    const float ms = (sMisc[0] + sMisc[1]) * (1.0f / kD);
                    const float rstd = 1.0f / sqrtf(ms + a.eps_norm);
                    y = nwj * (oj * rstd) * silu(bf16_to_f32(*slot));
                }
                *slot = f32_to_bf16(y);
            }
        }
        if (kPF) {
#pragma unroll
            for (int m = 0; m < kRows; ++m) S[m] = Sn[m];
        }
    }
    // the outputs of every head and token: [hr][t][128] -> o rows
    lds_barrier();
    for (int i = tid; i < r * T * (kD / 8); i += kThreads) {
        const int hr = i / (T * 16), t = (i / 16) % T, j8 = i % 16;
        *reinterpret_cast<uint4 *>(a.o + (((size_t)b * T + t) * a.Hv + kh * r + hr) * kD + j8 * 8) =
            *reinterpret_cast<const uint4 *>(sZ + i * 8);
    }
}

} // namespace

size_t decode_lds_bytes(int T, int r) { return sizeof(float) * (size_t)DecodeLds(T, r).total; }

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
    static_assert(kMaxTokens == 8, "kernel variants cover 1, 2, 4 and 8 tokens");
    const void *fn = p.T == 1   ? reinterpret_cast<const void *>(decode_kernel<1>)
                     : p.T == 2 ? reinterpret_cast<const void *>(decode_kernel<2>)
                     : p.T <= 4 ? reinterpret_cast<const void *>(decode_kernel<4>)
                                : reinterpret_cast<const void *>(decode_kernel<8>);
    if (lds > 64 * 1024) {  // beyond the default dynamic LDS limit: raise it for this kernel
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return fail("hipFuncSetAttribute(decode_kernel)", e);
    }
    void *args[] = {&a};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(p.B * p.Hk)), dim3(kThreads), args, lds, stream);
    return e == hipSuccess ? 0 : fail("hipLaunchKernel(decode_kernel)", e);
}

} // namespace gdn
