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
//  chunk_prep_kernel  one workgroup per (sequence, chunk, key head), all in
//                     parallel.  conv + SiLU + L2 norm (+ 1/sqrt(128) on q) of
//                     the chunk's q/k rows -> fp16 q^, k^; Q K^T and K K^T
//                     once per key head; then for each of its r value heads
//                     the decays, T = (I + L)^{-1} (16x16 diagonal blocks by
//                     substitution in fp32, the rest as block products on
//                     MFMA), T diag(beta) and P = (Q K^T) o R as packed lower
//                     16x16 blocks.  Everything that does not depend on the
//                     state is done here, once, instead of inside the
//                     sequential loop of every value slice.
//  chain_kernel<NT>   one workgroup (4 waves, one per SIMD) per (sequence, value head,
//                     slice of 16*NT value columns); state columns evolve
//                     independently, so a head splits into 8/NT slices on
//                     different CUs.  Waves 0..NT-1 each own one 16-column
//                     tile of the state in MFMA accumulator registers and run
//                     the chunk loop -- the only sequential dependency -- with
//                     no LDS round trip or barrier inside a chunk: the
//                     accumulator layout of two adjacent 16-row tiles is the
//                     B-operand layout of a 16x16x32 MFMA under one fixed
//                     permutation of k, applied to the A operand as well.  The
//                     other waves convert v (conv + SiLU) for the next chunk
//                     and apply the gated RMSNorm to the previous chunk.
//                     Operands of chunk c+1 are fetched into registers while
//                     chunk c runs.  The norm needs all 128 columns of a row:
//                     every 16-column tile publishes per-row sums of squares
//                     as tagged 64-bit words (value | chunk tag) and the
//                     helpers read all of them two chunks later.  Slices are
//                     handed out from per-XCD ticket queues in the order
//                     workgroups start, so a slice only ever waits for
//                     siblings that are running or next in line; every wait
//                     is bounded.
// All contractions use fp16 MFMA operands with fp32 accumulation; the state is
// carried in fp32 across chunks; inputs and outputs are bf16.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kD = 128;        // head width
constexpr int kC = 64;         // chunk length
// Chunks of partial sums kept per tile.  A slice reads chunk c-3 in iteration
// c, and a sibling cannot finish iteration c+2 before this slice has published
// chunk c-1, so the newest chunk a sibling can be writing meanwhile is c+1: five
// chunks live at once, eight slots keep the index a power of two.
constexpr int kRing = 8;
constexpr int kTiles = 8;      // 16-column tiles per head
constexpr uint32_t kSpinLimit = 1u << 20;  // bound of every cross-workgroup wait (~0.3 s)

// LDS pitches (elements) so that 16-row MFMA fragment reads hit distinct banks.
constexpr int P128 = kD + 8;   // fp16 rows of 128
constexpr int P64 = kC + 8;    // fp16 rows of 64
constexpr int PL = kC + 4;     // fp32 rows of 64
constexpr int PTD = 20;        // fp32 rows of a 16x16 block

// Workspace blocks (in fp16 elements).  Matrices that the chain kernel reads
// as MFMA A operands are stored with their contraction index permuted inside
// every 32-wide block, so that each lane's eight k-values (original indices
// 4q..4q+3 and 16+4q..16+4q+3, matching the accumulator layout of two
// adjacent 16-row tiles) are contiguous: stored position p holds original
// index 4*(p>>3) + (p&3) + 16*((p>>2)&1).  kpos(m) is where the original
// 4-group m (indices 4m..4m+3) of a 32-block starts.
constexpr int kBlk = 256;                              // one 16x16 block (prep staging)
constexpr int kQK = 2 * kC * kD;                       // q^ [64][128], k^ [64][128] (keys permuted)
constexpr int kTri = 32 * 32 + 32 * 64;                // lower triangle at 32-granularity: rows 0-31 x 32, rows 32-63 x 64
constexpr int kTP = 2 * kTri + 2 * 2 * kC;             // T diag(beta), P (tokens permuted), then 2 x 64 fp32
constexpr int kTPVec = 2 * kTri;                       // offset of the fp32 decay vectors

__host__ __device__ constexpr int kpos(int m) { return m < 4 ? 8 * m : 8 * (m - 4) + 4; }

__device__ __forceinline__ void tri_block(int blk, int &bi, int &bj) {
    bi = blk < 1 ? 0 : blk < 3 ? 1 : blk < 6 ? 2 : 3;
    bj = blk - bi * (bi + 1) / 2;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Accumulator tiles a (rows 4q..4q+3 of a 16-row tile) and b (the next tile)
// as one 8-element MFMA B operand, in the permuted k order described above.
__device__ __forceinline__ half8 pack_tiles(const floatx4 &a, const floatx4 &b) {
    return half8{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3],
                 (_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
}

// ========================================================================
// chunk_prep_kernel
// ========================================================================

struct PrepArgs {
    const uint16_t *q, *k, *conv_w, *conv_state_in;
    const float *g, *beta;
    uint16_t *conv_state_out;
    _Float16 *qkw;  // [B][nch][Hk][kQK]
    _Float16 *tpw;  // [B][nch][Hv][kTP]
    int B, T, Hk, Hv, r, Cc, conv, nch;
    float eps_l2;
};

struct PrepLds {
    static constexpr size_t sQ = 0;                        // fp16 [64][P128]
    static constexpr size_t sK = sQ + 2 * kC * P128;       // fp16 [64][P128]
    static constexpr size_t sL = sK + 2 * kC * P128;       // fp32 [64][PL]
    static constexpr size_t sTd = sL + 4 * kC * PL;        // fp32 [4][16][PTD]
    static constexpr size_t sT16T = sTd + 4 * 4 * 16 * PTD;  // fp16 [64][P64]  T transposed
    static constexpr size_t sPst = sT16T + 2 * kC * P64;   // fp16 [10][256]  P staging
    static constexpr size_t sTbst = sPst + 2 * 10 * kBlk;  // fp16 [10][256]  T diag(beta) staging
    static constexpr size_t sG = sTbst + 2 * 10 * kBlk;    // fp32 [64]
    static constexpr size_t sB = sG + 4 * kC;              // fp32 [64]
    static constexpr size_t bytes = sB + 4 * kC;
};

// grid (nch, Hk, B), 256 threads
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrepArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    _Float16 *sQ = reinterpret_cast<_Float16 *>(smem + PrepLds::sQ);
    _Float16 *sK = reinterpret_cast<_Float16 *>(smem + PrepLds::sK);
    float *sL = reinterpret_cast<float *>(smem + PrepLds::sL);
    float *sTd = reinterpret_cast<float *>(smem + PrepLds::sTd);
    _Float16 *sT16T = reinterpret_cast<_Float16 *>(smem + PrepLds::sT16T);
    _Float16 *sPst = reinterpret_cast<_Float16 *>(smem + PrepLds::sPst);
    _Float16 *sTbst = reinterpret_cast<_Float16 *>(smem + PrepLds::sTbst);
    float *sG = reinterpret_cast<float *>(smem + PrepLds::sG);
    float *sB = reinterpret_cast<float *>(smem + PrepLds::sB);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, lq = lane >> 4;
    const int c = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
    const int tc0 = c * kC;
    _Float16 *qkb = a.qkw + (((size_t)b * a.nch + c) * a.Hk + kh) * kQK;

    // ---- 1. q/k rows: conv + SiLU + L2 norm.  Thread = (4-token segment, q|k, 8 channels)
    {
        const int cg = tid & 15, m = (tid >> 4) & 1;
        const uint16_t *src = m ? a.k : a.q;
        const int ch = m * a.Hk * kD + kh * kD + cg * 8;  // conv channel of element 0
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
        const float qscale = m ? 1.0f : 0.08838834764831845f;  // 1/sqrt(128) on q
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tl0 = ((tid >> 5) + 8 * u) * 4;  // local token of the segment
            float x[7][8];
#pragma unroll
            for (int rr = 0; rr < 7; ++rr) {
                const int t = tc0 + tl0 - 3 + rr;
                uint4 raw = make_uint4(0, 0, 0, 0);
                if (t >= 0 && t < a.T)
                    raw = *reinterpret_cast<const uint4 *>(src + (((size_t)b * a.T + t) * a.Hk + kh) * kD + cg * 8);
                else if (t < 0 && a.conv && a.conv_state_in)
                    raw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + (3 + t)) * a.Cc + ch);
                unpack_bf16x8(raw, x[rr]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float uu[8];
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uu[e] = a.conv ? silu(w[e][0] * x[i][e] + w[e][1] * x[i + 1][e] + w[e][2] * x[i + 2][e] +
                                          w[e][3] * x[i + 3][e])
                                   : x[i + 3][e];
                    ss += uu[e] * uu[e];
                }
                ss = group_sum<16>(ss);
                const bool valid = tc0 + tl0 + i < a.T;
                const float sc = valid ? qscale / sqrtf(ss + a.eps_l2) : 0.0f;  // rows past T are zero
                half8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    hv[e] = static_cast<_Float16>(uu[e] * sc);
                }
                const int row = tl0 + i;
                *reinterpret_cast<half8 *>((m ? sK : sQ) + row * P128 + cg * 8) = hv;
                _Float16 *gdst = qkb + m * kC * kD + row * kD + 32 * (cg >> 2);
                const int g2 = 2 * (cg & 3);  // original 4-groups g2, g2+1 of this 32-block
                *reinterpret_cast<half4 *>(gdst + kpos(g2)) = half4{hv[0], hv[1], hv[2], hv[3]};
                *reinterpret_cast<half4 *>(gdst + kpos(g2 + 1)) = half4{hv[4], hv[5], hv[6], hv[7]};
            }
        }
        // raw q/k inputs of the last three tokens -> conv state out
        if (c == 0 && a.conv && a.conv_state_out && tid < 96) {
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
    lds_barrier();

    // ---- 2. raw K K^T and Q K^T lower tiles, kept in registers (5 tasks per wave)
    floatx4 raw[5];
#pragma unroll
    for (int u = 0; u < 5; ++u) {
        const int task = wave + 4 * u;
        const bool isP = task >= 10;
        const int tt = isP ? task - 10 : task;
        int ti, tj;
        tri_block(tt, ti, tj);
        const _Float16 *Aop = isP ? sQ : sK;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const half8 av = lds_half8(Aop + (16 * ti + l16) * P128 + 32 * ks + 8 * lq);
            const half8 bv = lds_half8(sK + (16 * tj + l16) * P128 + 32 * ks + 8 * lq);
            acc = mfma16x16x32(av, bv, acc);
        }
        raw[u] = acc;
    }
    lds_barrier();

    // ---- 3. per value head of this key head
    for (int hr = 0; hr < a.r; ++hr) {
        const int h = kh * a.r + hr;
        _Float16 *tpb = a.tpw + (((size_t)b * a.nch + c) * a.Hv + h) * kTP;
        if (wave == 0) {
            const int t = tc0 + lane;
            const bool valid = t < a.T;
            const size_t gi = ((size_t)b * a.T + (valid ? t : 0)) * a.Hv + h;
            float gv = valid ? a.g[gi] : 0.0f;
            const float bv = valid ? a.beta[gi] : 0.0f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float t2 = __shfl_up(gv, o, 64);
                if (lane >= o) gv += t2;
            }
            const float gc = __shfl(gv, 63, 64);
            sG[lane] = gv;
            sB[lane] = bv;
            float *vec = reinterpret_cast<float *>(tpb + kTPVec);
            vec[lane] = __expf(gv);
            vec[kC + lane] = __expf(gc - gv);
        }
        lds_barrier();

        // L (fp32, strictly lower) and P (fp16 staging, lower incl. diagonal)
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int task = wave + 4 * u;
            const bool isP = task >= 10;
            const int tt = isP ? task - 10 : task;
            int ti, tj;
            tri_block(tt, ti, tj);
            const int col = 16 * tj + l16;
            const float gcol = sG[col];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * ti + 4 * lq + e;
                const float rdec = __expf(sG[row] - gcol);
                if (isP)
                    sPst[tt * kBlk + (4 * lq + e) * 16 + l16] =
                        static_cast<_Float16>(col <= row ? raw[u][e] * rdec : 0.0f);
                else
                    sL[row * PL + col] = col < row ? sB[row] * raw[u][e] * rdec : 0.0f;
            }
        }
        lds_barrier();

        // diagonal 16x16 blocks of T = (I + L)^{-1}: forward substitution, one column per lane
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
            const int db = wave * (wave + 1) / 2 + wave;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                sTd[(wave * 16 + rr) * PTD + cidx] = x[rr];
                sT16T[(w0 + cidx) * P64 + w0 + rr] = static_cast<_Float16>(x[rr]);
                sTbst[db * kBlk + rr * 16 + cidx] = static_cast<_Float16>(x[rr] * bc);
            }
        }
        lds_barrier();

        // off-diagonal blocks, column block J = wave: T_IJ = -T_II sum_{K=J}^{I-1} L_IK T_KJ
        if (wave < 3) {
            const int J = wave;
            const float bcol = sB[16 * J + l16];
            for (int I = J + 1; I < 4; ++I) {
                floatx4 y = {0.f, 0.f, 0.f, 0.f};
                for (int K = J; K < I; ++K) {
                    half4 av;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        av[e] = static_cast<_Float16>(sL[(16 * I + l16) * PL + 16 * K + 4 * lq + e]);
                    const half4 bv = lds_half4(sT16T + (16 * J + l16) * P64 + 16 * K + 4 * lq);
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
                const int blk = I * (I + 1) / 2 + J;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    th[e] = static_cast<_Float16>(-t[e]);
                    sTbst[blk * kBlk + (4 * lq + e) * 16 + l16] = static_cast<_Float16>(-t[e] * bcol);
                }
                *reinterpret_cast<half4 *>(sT16T + (16 * J + l16) * P64 + 16 * I + 4 * lq) = th;
                wave_lds_sync();
            }
        }
        lds_barrier();

        // T diag(beta) and P to the workspace: lower triangle at 32-granularity, tokens
        // (columns) permuted inside 32-blocks; 8-byte groups of 4 columns
        for (int idx = tid; idx < 2 * kTri / 4; idx += 256) {
            const int mat = idx >= kTri / 4, j = mat ? idx - kTri / 4 : idx;
            int r, cb, m, dst;
            if (j < 256) {
                r = j >> 3, cb = 0, m = j & 7;
                dst = r * 32 + kpos(m);
            } else {
                const int j2 = j - 256;
                r = 32 + (j2 >> 4), cb = (j2 >> 3) & 1, m = j2 & 7;
                dst = 32 * 32 + (r - 32) * 64 + 32 * cb + kpos(m);
            }
            const int oc = 32 * cb + 4 * m;  // first original column of the group
            half4 v4 = {0, 0, 0, 0};
            if ((oc >> 4) <= (r >> 4)) {
                const int blk = (r >> 4) * ((r >> 4) + 1) / 2 + (oc >> 4);
                v4 = *reinterpret_cast<const half4 *>((mat ? sPst : sTbst) + blk * kBlk + (r & 15) * 16 + (oc & 15));
            }
            *reinterpret_cast<half4 *>(tpb + mat * kTri + dst) = v4;
        }
        lds_barrier();
    }
}

// ========================================================================
// chain_kernel<NT>
// ========================================================================

struct ChainArgs {
    const _Float16 *qkw, *tpw;
    const uint16_t *v, *z, *conv_w, *norm_w, *conv_state_in;
    const float *state_in;
    uint16_t *o, *conv_state_out;
    float *state_out;
    unsigned long long *mbox;  // [B*Hv][kTiles][kRing][64]: per-row sums of squares of each slice
    unsigned int *counters;    // [B*Hv]
    unsigned int *err;
    unsigned int *tickets;     // [8] next item of each XCD queue
    unsigned int *exits;       // workgroups that have left the item loop
    int B, T, Hk, Hv, r, Cc, conv, norm, nch, n_items, grid;
    float eps_norm;
};

template <int NT>
struct ChainLds {
    static constexpr int BV = 16 * NT;
    static constexpr int PV = BV + 4;
    static constexpr size_t sQ = 0;                          // fp16 [64][P128]   q^
    static constexpr size_t sK = sQ + 2 * kC * P128;         // fp16 [64][P128]   k^
    static constexpr size_t sKT = sK + 2 * kC * P128;        // fp16 [128][P64]   k^T
    static constexpr size_t sTb = sKT + 2 * kD * P64;        // fp16 [64][P64]    T diag(beta)
    static constexpr size_t sP = sTb + 2 * kC * P64;         // fp16 [64][P64]    (Q K^T) o R
    static constexpr size_t sEG = sP + 2 * kC * P64;         // fp32 [64] e^G, then [64] e^{G_C - G}
    static constexpr size_t sV = sEG + 4 * 2 * kC;           // fp32 [2][64][PV]  conv(v) of the slice
    static constexpr size_t sO = sV + 4 * 2 * kC * PV;       // fp32 [5][64][PV]  pre-norm output
    static constexpr size_t sRawV = sO + 4 * 5 * kC * PV;    // bf16 [2][64][BV]  raw v of the slice
    static constexpr size_t sZ = sRawV + 2 * 2 * kC * BV;    // bf16 [64][BV]     z of the slice
    static constexpr size_t sRstd = sZ + 2 * kC * BV;        // fp32 [2][64]      gated-norm 1/rms per row
    static constexpr size_t sCW = sRstd + 4 * 2 * kC;        // fp32 [BV][4]      conv taps of the slice's v channels
    static constexpr size_t sNW = sCW + 4 * 4 * BV;          // fp32 [BV]         gated-norm weights of the slice
    static constexpr size_t bytes = sNW + 4 * BV;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Global data of one pipeline step, fetched by the helper waves into registers
// while the chain waves compute: the chunk's operands (q^, k^ [64][128]: 2048
// 16-byte pieces contiguous in the workspace; T diag(beta), P: 384 pieces
// each; the decay vectors: 32 pieces), a later chunk's raw v slice and an
// earlier chunk's z slice (8*BV pieces each).  k^T is rebuilt in LDS.

template <int NT>
struct PF {
    static constexpr int BV = 16 * NT;
    static constexpr int NH = (4 - NT) * 64;          // helper threads
    static constexpr int NV = 8 * BV;                 // 16-byte pieces of one 64-row slice
    static constexpr int NQK = (2048 + NH - 1) / NH;  // q^, k^ pieces per helper
    static constexpr int NTP = (800 + NH - 1) / NH;   // T diag(beta), P, decay-vector pieces per helper
    static constexpr int NVZ = (NV + NH - 1) / NH;    // raw-v (and z) pieces per helper
};

// Registers of one pipeline step (helpers).
template <int NT>
struct Stage {
    u32x4 qk[PF<NT>::NQK], tp[PF<NT>::NTP], rv[PF<NT>::NVZ], z[PF<NT>::NVZ];
};

// Issue the loads of one pipeline step: operands of chunk c_op, raw v of chunk
// c_v, z of chunk c_z.  Rows of chunks outside [0, nch) or past T are read from
// a valid row and zeroed when stored, so issuing never waits for a load.
template <int NT>
__device__ __forceinline__ void prefetch_issue(const ChainArgs &a, int b, int h, int kh, int sv0, int c_op, int c_v,
                                               int c_z, int htid, Stage<NT> &st) {
    using F = PF<NT>;
    constexpr int NCG = F::BV / 8;
    const int cop = min(c_op, a.nch - 1);
    const u32x4 *qk = reinterpret_cast<const u32x4 *>(a.qkw + (((size_t)b * a.nch + cop) * a.Hk + kh) * kQK) + htid;
    // (pieces past the end re-read the last one)
    const u32x4 *tp = reinterpret_cast<const u32x4 *>(a.tpw + (((size_t)b * a.nch + cop) * a.Hv + h) * kTP);
#pragma unroll
    for (int u = 0; u < F::NQK; ++u) st.qk[u] = qk[min(F::NH * u, 2047 - htid)];
#pragma unroll
    for (int u = 0; u < F::NTP; ++u) st.tp[u] = tp[min(htid + F::NH * u, 799)];
    const int cg = htid % NCG;
    const uint16_t *zsrc = a.norm ? a.z : a.v;
#pragma unroll
    for (int u = 0; u < F::NVZ; ++u) {
        const int row = min((htid + F::NH * u) / NCG, kC - 1);
        const int tv = min(max(c_v, 0) * kC + row, a.T - 1), tz = min(max(c_z, 0) * kC + row, a.T - 1);
        st.rv[u] = *reinterpret_cast<const u32x4 *>(a.v + (((size_t)b * a.T + tv) * a.Hv + h) * kD + sv0 + 8 * cg);
        st.z[u] = *reinterpret_cast<const u32x4 *>(zsrc + (((size_t)b * a.T + tz) * a.Hv + h) * kD + sv0 + 8 * cg);
    }
}

// Store one pipeline step's registers into LDS: operands, raw v into buffer
// rv_buf, z.
template <int NT>
__device__ __forceinline__ void prefetch_store(unsigned char *smem, int htid, int rv_buf, int c_v, int c_z, int T,
                                               const Stage<NT> &st) {
    using L = ChainLds<NT>;
    using F = PF<NT>;
    _Float16 *sQ = reinterpret_cast<_Float16 *>(smem + L::sQ);
    _Float16 *sTb = reinterpret_cast<_Float16 *>(smem + L::sTb);
    // q^ then k^ (both [64][P128], adjacent)
#pragma unroll
    for (int u = 0; u < F::NQK; ++u) {
        const int i = htid + F::NH * u;
        if (i < 2048) *reinterpret_cast<u32x4 *>(sQ + (i >> 4) * P128 + (i & 15) * 8) = st.qk[u];
    }
    // T diag(beta) then P (both [64][P64], adjacent), then the decay vectors
#pragma unroll
    for (int u = 0; u < F::NTP; ++u) {
        const int i = htid + F::NH * u;
        if (i < 768) {
            const int j = i % 384;
            const int off = (i >= 384 ? kC * P64 : 0) +
                            (j < 128 ? (j >> 2) * P64 + (j & 3) * 8 : (32 + ((j - 128) >> 3)) * P64 + ((j - 128) & 7) * 8);
            *reinterpret_cast<u32x4 *>(sTb + off) = st.tp[u];
        } else if (i < 800) {
            reinterpret_cast<u32x4 *>(smem + L::sEG)[i - 768] = st.tp[u];
        }
    }
    u32x4 *sRawV = reinterpret_cast<u32x4 *>(smem + L::sRawV) + rv_buf * F::NV;
    u32x4 *sZ = reinterpret_cast<u32x4 *>(smem + L::sZ);
    constexpr int NCG = F::BV / 8;
#pragma unroll
    for (int u = 0; u < F::NVZ; ++u) {
        const int i = htid + F::NH * u;
        if (i < F::NV) {
            const int row = i / NCG;
            const bool okv = c_v >= 0 && c_v * kC + row < T, okz = c_z >= 0 && c_z * kC + row < T;
            sRawV[i] = okv ? st.rv[u] : u32x4{0u, 0u, 0u, 0u};
            sZ[i] = okz ? st.z[u] : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// k^T in LDS from k^ (helpers): sKT[d][tpos] = sK[t][kpos], where both axes
// keep their 32-block permutation of the stored contraction index.  A unit is
// 4 consecutive tokens x one 4-group of keys (contiguous in both layouts).
template <int NT>
__device__ __forceinline__ void transpose_k(unsigned char *smem, int htid) {
    using L = ChainLds<NT>;
    const _Float16 *sK = reinterpret_cast<const _Float16 *>(smem + L::sK);
    _Float16 *sKT = reinterpret_cast<_Float16 *>(smem + L::sKT);
    constexpr int NH = (4 - NT) * 64;
    for (int unit = htid; unit < 16 * 32; unit += NH) {
        const int tg = unit & 15, kg = unit >> 4;  // token 4-group (0..15), key 4-group (0..31)
        // stored positions: key 4-group kg of block kg/8 sits at 32*(kg/8) + kpos(kg%8); same for tokens
        const int kp = 32 * (kg >> 3) + kpos(kg & 7), tp = 32 * (tg >> 3) + kpos(tg & 7);
        half4 r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = lds_half4(sK + (4 * tg + i) * P128 + kp);
        // natural key index of stored position kp+j: 4*kg + j
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<half4 *>(sKT + (4 * kg + j) * P64 + tp) = half4{r[0][j], r[1][j], r[2][j], r[3][j]};
    }
}

__device__ __forceinline__ unsigned long long spin_load(unsigned long long *p, uint32_t tag, unsigned int *err,
                                                        int &broken) {
    // Wait until the tagged word at p carries `tag`.  Bounded: on a timeout the
    // error word is raised and this thread stops waiting for the rest of the
    // launch, so a lost sibling cannot stall every later chunk.
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

// One chunk of the state chain for one 16-column tile (chain waves), first
// part: K S, X, Delta, O (to sOc).  S holds the tile in the accumulator layout
// (key-row tiles ti = 0..7).  Every MFMA A operand is a single 16-byte LDS read
// thanks to the permuted storage of the contraction index.
template <int NT>
__device__ __forceinline__ void chain_chunk_a(unsigned char *smem, const floatx4 (&S)[8], const float *sVc,
                                              float *sOc, int jc, int l16, int lq, half8 (&Dsb)[2]) {
    using L = ChainLds<NT>;
    constexpr int PV = L::PV;
    const _Float16 *sQ = reinterpret_cast<const _Float16 *>(smem + L::sQ);
    const _Float16 *sK = reinterpret_cast<const _Float16 *>(smem + L::sK);
    const _Float16 *sTb = reinterpret_cast<const _Float16 *>(smem + L::sTb);
    const _Float16 *sP = reinterpret_cast<const _Float16 *>(smem + L::sP);
    const float *sEG = reinterpret_cast<const float *>(smem + L::sEG);
    const float *sEGC = sEG + kC;

    half8 Sb[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) Sb[s2] = pack_tiles(S[2 * s2], S[2 * s2 + 1]);

    half8 fr[16];  // A-operand fragments of one phase, loaded together
    // K S (token-row tiles I, contraction over key dims), then X = V - e^G K S
#pragma unroll
    for (int f = 0; f < 16; ++f) fr[f] = lds_half8(sK + (16 * (f >> 2) + l16) * P128 + 32 * (f & 3) + 8 * lq);
    floatx4 X[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        floatx4 ks = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) ks = mfma16x16x32(fr[4 * I + s2], Sb[s2], ks);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * I + 4 * lq + e;
            X[I][e] = sVc[row * PV + jc] - sEG[row] * ks[e];
        }
    }
    const half8 Xb[2] = {pack_tiles(X[0], X[1]), pack_tiles(X[2], X[3])};

    // Delta = T diag(beta) X  (lower triangular: 32-row block s2 uses k-steps <= s2)
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        const int s2 = f < 2 ? 0 : 1, hh = f < 2 ? f : (f - 2) >> 1, k2 = f < 2 ? 0 : (f - 2) & 1;
        fr[f] = lds_half8(sTb + (32 * s2 + 16 * hh + l16) * P64 + 32 * k2 + 8 * lq);
    }
    half8 Db[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
        if (s2 == 0) {
            d0 = mfma16x16x32(fr[0], Xb[0], d0);
            d1 = mfma16x16x32(fr[1], Xb[0], d1);
        } else {
            d0 = mfma16x16x32(fr[2], Xb[0], d0);
            d0 = mfma16x16x32(fr[3], Xb[1], d0);
            d1 = mfma16x16x32(fr[4], Xb[0], d1);
            d1 = mfma16x16x32(fr[5], Xb[1], d1);
        }
        Db[s2] = pack_tiles(d0, d1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Dsb[s2][e] = static_cast<_Float16>(d0[e] * sEGC[32 * s2 + 4 * lq + e]);
            Dsb[s2][4 + e] = static_cast<_Float16>(d1[e] * sEGC[32 * s2 + 16 + 4 * lq + e]);
        }
    }

    // O = e^G Q S + P Delta
#pragma unroll
    for (int f = 0; f < 16; ++f) fr[f] = lds_half8(sQ + (16 * (f >> 2) + l16) * P128 + 32 * (f & 3) + 8 * lq);
    half8 fp[6];
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        const int I = f < 2 ? f : 2 + ((f - 2) >> 1), s2 = f < 2 ? 0 : (f - 2) & 1;
        fp[f] = lds_half8(sP + (16 * I + l16) * P64 + 32 * s2 + 8 * lq);
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        floatx4 qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) qs = mfma16x16x32(fr[4 * I + s2], Sb[s2], qs);
        floatx4 ot;
#pragma unroll
        for (int e = 0; e < 4; ++e) ot[e] = qs[e] * sEG[16 * I + 4 * lq + e];
        if (I < 2) {
            ot = mfma16x16x32(fp[I], Db[0], ot);
        } else {
            ot = mfma16x16x32(fp[2 + 2 * (I - 2)], Db[0], ot);
            ot = mfma16x16x32(fp[3 + 2 * (I - 2)], Db[1], ot);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sOc[(16 * I + 4 * lq + e) * PV + jc] = ot[e];
    }

}

// Second part: S = e^{G_C} S + K^T Delta~  (key-row tiles ti, contraction over
// tokens).  Needs k^T of the chunk in LDS.
template <int NT>
__device__ __forceinline__ void chain_chunk_b(unsigned char *smem, floatx4 (&S)[8], const half8 (&Dsb)[2], int l16,
                                              int lq) {
    using L = ChainLds<NT>;
    const _Float16 *sKT = reinterpret_cast<const _Float16 *>(smem + L::sKT);
    const float *sEG = reinterpret_cast<const float *>(smem + L::sEG);
    half8 fr[16];
#pragma unroll
    for (int f = 0; f < 16; ++f) fr[f] = lds_half8(sKT + (16 * (f >> 1) + l16) * P64 + 32 * (f & 1) + 8 * lq);
    const float dC = sEG[kC - 1];
#pragma unroll
    for (int ti = 0; ti < 8; ++ti) {
        floatx4 acc = S[ti] * dC;
        acc = mfma16x16x32(fr[2 * ti], Dsb[0], acc);
        acc = mfma16x16x32(fr[2 * ti + 1], Dsb[1], acc);
        S[ti] = acc;
    }
}

template <int NT>
__global__ __launch_bounds__(256) void chain_kernel(ChainArgs a) {
    using L = ChainLds<NT>;
    using F = PF<NT>;
    constexpr int BV = L::BV, PV = L::PV;
    constexpr int NSL = kTiles / NT;
    constexpr int NCG = BV / 8;  // 8-column groups per slice row
    constexpr int NH = F::NH;    // helper threads
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float *sV = reinterpret_cast<float *>(smem + L::sV);
    float *sO = reinterpret_cast<float *>(smem + L::sO);
    const uint16_t *sRawV = reinterpret_cast<const uint16_t *>(smem + L::sRawV);
    const uint16_t *sZ = reinterpret_cast<const uint16_t *>(smem + L::sZ);
    float *sRstd = reinterpret_cast<float *>(smem + L::sRstd);
    float *sCW = reinterpret_cast<float *>(smem + L::sCW);
    float *sNW = reinterpret_cast<float *>(smem + L::sNW);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: role branches are scalar
    const int l16 = lane & 15, lq = lane >> 4;
    const bool is_chain = wave < NT;
    const int htid = tid - NT * 64;                       // helper index
    const int hcg = (htid >= 0 ? htid : 0) % NCG;         // fixed column group of a helper (NH % NCG == 0)

    int broken = 0;
    __shared__ int s_item;
    // Work items (chain, slice) come from eight queues, one per XCD: chain c
    // sits in queue c % 8 and its slices are consecutive tickets.  A workgroup
    // serves the queue of the XCD it runs on (the slices of a chain then share
    // that XCD's L2), and the other queues once its own is empty.  Tickets are
    // taken only when a workgroup starts an item, so the items begun form a
    // prefix of every queue: the slices a workgroup waits for are either
    // running or next in line for the next free workgroup, and no launch-wide
    // co-residency is needed.
    const int xcc = static_cast<int>(xcc_id() & 7u);
    const int n_chains = a.B * a.Hv;
    int qi = 0;

    for (;;) {
        if (tid == 0) {
            int item = -1;
            for (; qi < 8 && item < 0; ) {
                const int q = (xcc + qi) & 7;
                const int nq = n_chains > q ? (n_chains - q + 7) / 8 : 0;
                const unsigned int t = __hip_atomic_fetch_add(a.tickets + q, 1u, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT);
                if (t < (unsigned int)(nq * NSL))
                    item = (q + 8 * (int)(t / NSL)) * NSL + (int)(t % NSL);
                else
                    ++qi;
            }
            s_item = item;
        }
        __syncthreads();
        const int item = s_item;
        __syncthreads();
        if (item < 0) break;
        const int chain = item / NSL, s = item % NSL;
        const int b = chain / a.Hv, h = chain % a.Hv, kh = h / a.r;
        const int sv0 = s * BV;
        const int jc = 16 * wave + l16;  // column of a chain-wave lane inside the slice
        const int hch = 2 * a.Hk * kD + h * kD + sv0 + hcg * 8;  // conv channel of a helper's 8 columns

        // conv + SiLU of the slice of v for chunk cc, from raw rows in LDS, into sV[cc & 1]
        auto conv_v = [&](int cc) {
            float *dst = sV + (cc & 1) * kC * PV;
            const uint16_t *cur = sRawV + (cc & 1) * kC * BV;
            const uint16_t *prev = sRawV + ((cc + 1) & 1) * kC * BV;  // chunk cc-1: the last three rows are the halo
            const float *hw = sCW + hcg * 8 * 4;                       // [8 channels][4 taps]
#pragma unroll 1
            for (int it = htid; it < kC * NCG; it += NH) {
                const int row = it / NCG;
                float x[4][8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r2 = row - 3 + j;
                    uint4 rw = make_uint4(0, 0, 0, 0);
                    if (j == 3 || a.conv) {
                        if (r2 >= 0)
                            rw = *reinterpret_cast<const uint4 *>(cur + r2 * BV + hcg * 8);
                        else if (cc > 0)
                            rw = *reinterpret_cast<const uint4 *>(prev + (kC + r2) * BV + hcg * 8);
                        else if (a.conv_state_in)
                            rw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + (3 + r2)) * a.Cc + hch);
                    }
                    unpack_bf16x8(rw, x[j]);
                }
                float u[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    u[e] = a.conv ? silu(hw[4 * e] * x[0][e] + hw[4 * e + 1] * x[1][e] + hw[4 * e + 2] * x[2][e] +
                                         hw[4 * e + 3] * x[3][e])
                                  : x[3][e];
                float4 *d4 = reinterpret_cast<float4 *>(dst + row * PV + hcg * 8);
                d4[0] = make_float4(u[0], u[1], u[2], u[3]);
                d4[1] = make_float4(u[4], u[5], u[6], u[7]);
            }
        };

        // ---- prologue: weights, operands of chunk 0, raw v of chunks 0 and 1, v of chunk 0
        if (htid >= 0 && htid < BV) {
            const int chn = 2 * a.Hk * kD + h * kD + sv0 + htid;
#pragma unroll
            for (int j = 0; j < 4; ++j) sCW[htid * 4 + j] = a.conv ? bf16_to_f32(a.conv_w[(size_t)chn * 4 + j]) : 0.0f;
            sNW[htid] = a.norm ? bf16_to_f32(a.norm_w[sv0 + htid]) : 1.0f;
        }
        if (!is_chain) {
            Stage<NT> st0;
            prefetch_issue<NT>(a, b, h, kh, sv0, 0, 0, -1, htid, st0);
            prefetch_store<NT>(smem, htid, 0, 0, -1, a.T, st0);
            prefetch_issue<NT>(a, b, h, kh, sv0, 0, 1, -1, htid, st0);  // (operands of chunk 0 again: harmless)
            prefetch_store<NT>(smem, htid, 1, 1, -1, a.T, st0);
        }
        lds_barrier();  // weights and raw v visible to every helper
        if (!is_chain) conv_v(0);
        lds_barrier();

        // ---- pipeline.  Chain waves and helpers run separate loops (the role test
        // is wave-uniform, so each wave takes one branch); both execute exactly
        // three barriers per iteration.  In iteration c the chain waves compute chunk c
        // into sO[c % 4]; the helpers publish the row sums of chunk c-1, finish the
        // norm statistics of chunk c-2, apply the norm to chunk c-3, convert v of
        // chunk c+1, and fetch the operands of chunk c+1, the raw v of chunk c+2
        // and the z of chunk c-2 -- every global access gets a full iteration --
        // and rebuild k^T of chunk c (needed by the chain's state update).
        const int last = a.nch + 3;
        if (is_chain) {
            floatx4 S[8];
            {
                const float *src = a.state_in ? a.state_in + (size_t)chain * kD * kD : nullptr;
#pragma unroll
                for (int ti = 0; ti < 8; ++ti)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[ti][e] = src ? src[(size_t)(16 * ti + 4 * lq + e) * kD + sv0 + jc] : 0.0f;
            }
            for (int c = 0; c <= last; ++c) {
                half8 Dsb[2];
                if (c < a.nch)
                    chain_chunk_a<NT>(smem, S, sV + (c & 1) * kC * PV, sO + (c % 5) * kC * PV, jc, l16, lq, Dsb);
                lds_barrier();  // k^T of chunk c built
                if (c < a.nch) chain_chunk_b<NT>(smem, S, Dsb, l16, lq);
                lds_barrier();  // chunk c done: operand buffers may be refilled
                lds_barrier();  // operands of chunk c+1 in place
            }
#pragma unroll
            for (int ti = 0; ti < 8; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.state_out[(size_t)chain * kD * kD + (size_t)(16 * ti + 4 * lq + e) * kD + sv0 + jc] = S[ti][e];
        } else {
            Stage<NT> pf;
            unsigned long long mbw[NSL];
            unsigned long long *mrow = a.mbox + (size_t)chain * kTiles * kRing * kC + htid;  // row htid (< 64)
            for (int c = 0; c <= last; ++c) {
                const bool fetch = c + 1 < a.nch || (c - 3 >= 0 && c - 3 < a.nch);
                // partial sums of chunk c-3 from every slice: issue now, use at the end
                const bool want_rstd = a.norm && htid < kC && c >= 3 && c - 3 < a.nch;
                if (want_rstd) {
#pragma unroll
                    for (int sib = 0; sib < NSL; ++sib)
                        mbw[sib] = __hip_atomic_load(mrow + ((size_t)sib * kRing + ((c - 3) % kRing)) * kC,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                if (fetch) prefetch_issue<NT>(a, b, h, kh, sv0, c + 1, c + 2, c - 3, htid, pf);
                if (c < a.nch) transpose_k<NT>(smem, htid);  // k^ of chunk c is in LDS
                lds_barrier();                                // k^T of chunk c built
                // row sums of chunk c-1 over this slice's columns -> mailbox
                if (a.norm && c >= 1 && c - 1 < a.nch && htid >= NH - kC) {
                    const int row = htid - (NH - kC);
                    const float *src = sO + ((c - 1) % 5) * kC * PV + row * PV;
                    float ss = 0.0f;
#pragma unroll
                    for (int j = 0; j < BV; j += 4) {
                        const float4 v4 = *reinterpret_cast<const float4 *>(src + j);
                        ss += v4.x * v4.x + v4.y * v4.y + v4.z * v4.z + v4.w * v4.w;
                    }
                    unsigned long long *mb =
                        a.mbox + (((size_t)chain * kTiles + s) * kRing + ((c - 1) % kRing)) * kC + row;
                    __hip_atomic_store(mb, ((unsigned long long)(uint32_t)c << 32) | __float_as_uint(ss),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                // gated RMSNorm + store of chunk c-4
                if (c >= 4 && c - 4 < a.nch) {
                    const int oc = c - 4;
                    const float *src = sO + (oc % 5) * kC * PV;
                    const float *rs = sRstd + (oc & 1) * kC;
#pragma unroll 1
                    for (int it = htid; it < kC * NCG; it += NH) {
                        const int row = it / NCG;
                        const int t = oc * kC + row;
                        if (t >= a.T) continue;
                        const float4 o0 = *reinterpret_cast<const float4 *>(src + row * PV + hcg * 8);
                        const float4 o1 = *reinterpret_cast<const float4 *>(src + row * PV + hcg * 8 + 4);
                        float y[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
                        if (a.norm) {
                            float zf[8];
                            unpack_bf16x8(*reinterpret_cast<const uint4 *>(sZ + row * BV + hcg * 8), zf);
                            const float rstd = rs[row];
#pragma unroll
                            for (int e = 0; e < 8; ++e) y[e] = sNW[hcg * 8 + e] * (y[e] * rstd) * silu(zf[e]);
                        }
                        *reinterpret_cast<uint4 *>(a.o + (((size_t)b * a.T + t) * a.Hv + h) * kD + sv0 + hcg * 8) =
                            pack_bf16x8(y);
                    }
                }
                if (c + 1 < a.nch) conv_v(c + 1);
                // 1/rms of chunk c-3's rows
                if (want_rstd) {
                    float tot = 0.0f;
#pragma unroll
                    for (int sib = 0; sib < NSL; ++sib) {
                        if ((uint32_t)(mbw[sib] >> 32) != (uint32_t)(c - 2))
                            mbw[sib] = spin_load(mrow + ((size_t)sib * kRing + ((c - 3) % kRing)) * kC,
                                                 (uint32_t)(c - 2), a.err, broken);
                        tot += __uint_as_float((uint32_t)mbw[sib]);
                    }
                    sRstd[((c - 3) & 1) * kC + htid] = 1.0f / sqrtf(tot * (1.0f / kD) + a.eps_norm);
                }
                lds_barrier();
                if (fetch) prefetch_store<NT>(smem, htid, c & 1, c + 2, c - 3, a.T, pf);
                lds_barrier();
            }
            // raw v inputs of the last three tokens -> conv state out
            if (a.conv && a.conv_state_out && htid < 3 * NCG) {
                const int sidx = htid / NCG, cg = htid % NCG;
                const int tau = a.T - 3 + sidx;
                const int ch = 2 * a.Hk * kD + h * kD + sv0 + cg * 8;
                uint4 rw = make_uint4(0, 0, 0, 0);
                if (tau >= 0)
                    rw = *reinterpret_cast<const uint4 *>(a.v + (((size_t)b * a.T + tau) * a.Hv + h) * kD + sv0 + cg * 8);
                else if (a.conv_state_in)
                    rw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + (3 + tau)) * a.Cc + ch);
                *reinterpret_cast<uint4 *>(a.conv_state_out + ((size_t)b * 3 + sidx) * a.Cc + ch) = rw;
            }
        }

        // ---- the last slice of a chain to finish clears the chain's mailbox
        if (a.norm) {
            __shared__ unsigned int last_one;
            if (tid == 0) {
                const unsigned int old =
                    __hip_atomic_fetch_add(a.counters + chain, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                last_one = (old == NSL - 1) ? 1u : 0u;
            }
            lds_barrier();
            if (last_one) {
                unsigned long long *mb = a.mbox + (size_t)chain * kTiles * kRing * kC;
                for (int i = tid; i < kTiles * kRing * kC; i += 256)
                    __hip_atomic_store(mb + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (tid == 0) __hip_atomic_store(a.counters + chain, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        lds_barrier();
    }
    // the last workgroup out rewinds the queues for the next launch
    if (tid == 0) {
        const unsigned int done =
            __hip_atomic_fetch_add(a.exits, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == (unsigned int)a.grid - 1) {
            for (int q = 0; q < 8; ++q) __hip_atomic_store(a.tickets + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.exits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int NT>
int launch_chain(const ChainArgs &base, hipStream_t stream) {
    ChainArgs a = base;
    constexpr size_t lds = ChainLds<NT>::bytes;
    auto fn = chain_kernel<NT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return fail("hipFuncSetAttribute(chain_kernel)", e);
    int dev = 0, ncu = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return fail("hipGetDevice", e);
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return fail("hipDeviceGetAttribute(multiprocessor count)", e);
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(fn), 256, lds)) !=
        hipSuccess)
        return fail("hipOccupancyMaxActiveBlocksPerMultiprocessor(chain_kernel)", e);
    constexpr int NSL = kTiles / NT;
    // One workgroup per resident slot at most: a workgroup that waits for its
    // sibling slices holds its slot, and the ticket order lets the next free
    // slot start them.  At least 8 * NSL slots keep a started slice of every
    // queue from blocking all slots.
    const int cap = ncu * per_cu;
    if (cap < 8 * NSL) return fail("chain_kernel: fewer resident workgroup slots than eight heads' slices");
    const int grid = a.n_items < cap ? a.n_items : cap;
    a.grid = grid;
    void *args[] = {&a};
    e = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(grid), dim3(256), args, lds, stream);
    return e == hipSuccess ? 0 : fail("hipLaunchKernel(chain_kernel)", e);
}

} // namespace

int plan_prefill(int B, int T, int Hk, int Hv, PrefillPlan *plan) {
    const long long chains = (long long)B * Hv;
    const int nsl = chains <= 32 ? 8 : 4;
    plan->nslice = nsl;
    plan->nt = kTiles / nsl;
    plan->bv = 16 * plan->nt;
    plan->nchunks = (T + kC - 1) / kC;
    plan->qk_bytes = align256((size_t)B * plan->nchunks * Hk * kQK * sizeof(_Float16));
    plan->tp_bytes = align256((size_t)B * plan->nchunks * Hv * kTP * sizeof(_Float16));
    plan->mbox_bytes = align256((size_t)chains * kTiles * kRing * kC * sizeof(unsigned long long)) +
                       align256((size_t)chains * sizeof(unsigned int)) + 256;
    plan->total_bytes = plan->qk_bytes + plan->tp_bytes + plan->mbox_bytes;
    return 0;
}

int launch_prefill(const PrefillParams &p, const PrefillPlan &plan, hipStream_t stream) {
    unsigned char *ws = static_cast<unsigned char *>(p.workspace);
    _Float16 *qkw = reinterpret_cast<_Float16 *>(ws);
    _Float16 *tpw = reinterpret_cast<_Float16 *>(ws + plan.qk_bytes);
    unsigned char *mb = ws + plan.qk_bytes + plan.tp_bytes;
    const size_t chains = (size_t)p.B * p.Hv;
    const size_t mbox_sz = align256(chains * kTiles * kRing * kC * sizeof(unsigned long long));
    unsigned int *counters = reinterpret_cast<unsigned int *>(mb + mbox_sz);
    // last 256 bytes: error word, then the eight queue tickets and the exit count
    unsigned int *err = reinterpret_cast<unsigned int *>(mb + mbox_sz + align256(chains * sizeof(unsigned int)));

    PrepArgs pa;
    pa.q = p.q; pa.k = p.k; pa.conv_w = p.conv_w; pa.conv_state_in = p.conv_state_in;
    pa.g = p.g; pa.beta = p.beta; pa.conv_state_out = p.conv_state_out;
    pa.qkw = qkw; pa.tpw = tpw;
    pa.B = p.B; pa.T = p.T; pa.Hk = p.Hk; pa.Hv = p.Hv; pa.r = p.Hv / p.Hk;
    pa.Cc = 2 * p.Hk * kD + p.Hv * kD; pa.conv = p.conv_width == 4; pa.nch = plan.nchunks;
    pa.eps_l2 = p.eps_l2;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(chunk_prep_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)PrepLds::bytes);
    if (e != hipSuccess) return fail("hipFuncSetAttribute(chunk_prep_kernel)", e);
    void *pargs[] = {&pa};
    e = hipLaunchKernel(reinterpret_cast<const void *>(chunk_prep_kernel),
                        dim3((unsigned)plan.nchunks, (unsigned)p.Hk, (unsigned)p.B), dim3(256), pargs, PrepLds::bytes,
                        stream);
    if (e != hipSuccess) return fail("hipLaunchKernel(chunk_prep_kernel)", e);

    ChainArgs a;
    a.qkw = qkw; a.tpw = tpw;
    a.v = p.v; a.z = p.z; a.conv_w = p.conv_w; a.norm_w = p.norm_w; a.conv_state_in = p.conv_state_in;
    a.state_in = p.state_in; a.o = p.o; a.conv_state_out = p.conv_state_out; a.state_out = p.state_out;
    a.mbox = reinterpret_cast<unsigned long long *>(mb); a.counters = counters; a.err = err;
    a.tickets = err + 16; a.exits = err + 32;
    a.B = p.B; a.T = p.T; a.Hk = p.Hk; a.Hv = p.Hv; a.r = pa.r; a.Cc = pa.Cc; a.conv = pa.conv; a.norm = p.norm;
    a.nch = plan.nchunks; a.n_items = (int)(chains * plan.nslice); a.grid = 0;
    a.eps_norm = p.eps_norm;
    switch (plan.nt) {
    case 1: return launch_chain<1>(a, stream);
    case 2: return launch_chain<2>(a, stream);
    default: return fail("prefill plan: unsupported value-tile count");
    }
}

} // namespace gdn
