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
// Kernels (all on the caller's stream, one after the other).
//  chunk_prep_kernel    one workgroup per (sequence, chunk, key head), all in
//                       parallel.  conv + SiLU + L2 norm (+ 1/sqrt(128) on q) of
//                       the chunk's q/k rows -> fp16 q^, k^ (and k^T); Q K^T and
//                       K K^T once per key head; then for each of its r value heads
//                       the decays, T = (I + L)^{-1} (16x16 diagonal blocks by
//                       substitution in fp32, the rest as block products on
//                       MFMA), T diag(beta) and P = (Q K^T) o R.  Everything
//                       that does not depend on the state is done here, once,
//                       instead of inside the sequential loop of every value
//                       slice.  Its outputs are written as MFMA operand
//                       fragments (64 lanes x 16 bytes each), so the later
//                       kernels load every operand straight into registers (or
//                       LDS) with one coalesced 1 KB load per fragment.  It also
//                       clears the workspace's exchange area.
//  pass_kernel<NT>      (gdn_pass.hip) the sequential pass over the chunks of every
//                       (sequence, value head), with the read-out and the gated
//                       RMSNorm.
//  Two-level scan, for few heads and long sequences (in place of pass_kernel):
//  segment_pass_kernel  every segment of a sequence on its own, from the identity
//                       and from zero (the segment map is affine in its start state);
//  seg_combine_kernel   the start state of every segment and the final state;
//  seg_output_kernel    the outputs from the segments' read-outs and start states,
//                       with the gated RMSNorm.
// All contractions use fp16 MFMA operands with fp32 accumulation; the state is
// carried in fp32 across chunks; inputs and outputs are bf16.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <mutex>

#include "gdn_internal.h"
#include "gdn_prefill_common.h"

namespace gdn {

namespace {


struct PrepArgs {
    const uint16_t *q, *k, *conv_w, *conv_state_in;
    const float *g, *beta;      // or the gate logits a, b when A_log is set
    const float *A_log, *dt_bias;
    uint16_t *conv_state_out;
    _Float16 *qkf;  // [B][nch][Hk][kQKF]
    _Float16 *tpf;  // [B][nch][Hv][kTPF]
    uint4 *clear;         // exchange area of the workspace, zeroed at the start of every call
    size_t clear_n16;     // its size in 16-byte units
    const int *cu;                     // packed sequences: [B + 1] token offsets (nullptr: even batch)
    int B, T, Hk, Hv, r, Cc, conv, nch;  // nch: chunks per sequence of an even batch
    float eps_l2;
};

// The q^/k^ tiles are dead once Q K^T and K K^T sit in registers, so the
// per-value-head buffers overlay them.
struct PrepLds {
    static constexpr size_t sQ = 0;                        // fp16 [64][P128]
    static constexpr size_t sK = sQ + 2 * kC * P128;       // fp16 [64][P128]
    static constexpr size_t sL = 0;                        // fp32 [64][PL]    (per value head from here on)
    static constexpr size_t sTd = sL + 4 * kC * PL;        // fp32 [4][16][PTD]
    static constexpr size_t sT16T = sTd + 4 * 4 * 16 * PTD;  // fp16 [64][P64]  T transposed
    static constexpr size_t sTbst = sT16T + 2 * kC * P64;  // fp16 [10][16][kTBS] T diag(beta) staging
    static constexpr size_t sGr = sTbst + 2 * 10 * kBlk;   // fp32 [r][64] g (then G), then [r][64] beta, of every value head
    static_assert(sGr >= sK + 2 * kC * P128, "g/beta staging must not overlay q^/k^");
    static size_t bytes(int r) { return sGr + 2 * 4 * (size_t)kC * r; }
};

// grid (slots * Hk), 256 threads: slot b nch + c of an even batch, else where seq_info places it.
// The sequential pass runs after this kernel on the same stream, so plain stores suffice.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void chunk_prep_kernel(PrepArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    _Float16 *sQ = reinterpret_cast<_Float16 *>(smem + PrepLds::sQ);
    _Float16 *sK = reinterpret_cast<_Float16 *>(smem + PrepLds::sK);
    float *sL = reinterpret_cast<float *>(smem + PrepLds::sL);
    float *sTd = reinterpret_cast<float *>(smem + PrepLds::sTd);
    _Float16 *sT16T = reinterpret_cast<_Float16 *>(smem + PrepLds::sT16T);
    _Float16 *sTbst = reinterpret_cast<_Float16 *>(smem + PrepLds::sTbst);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave bases stay scalar
    const int l16 = lane & 15, lq = lane >> 4;
    // blocks in chunk-major order: operand slot gc (chunk of a sequence, numbered sequence by
    // sequence), key head kh
    const int gc = blockIdx.x / a.Hk, kh = blockIdx.x % a.Hk;
    // the exchange area (error word, queue tickets, mailbox) starts every call at zero
    for (size_t i = (size_t)blockIdx.x * 256 + tid; i < a.clear_n16; i += (size_t)gridDim.x * 256)
        a.clear[i] = make_uint4(0, 0, 0, 0);
    const int b = a.cu ? find_seq(a.cu, a.B, gc, lane) : gc / a.nch;
    const SeqInfo si = seq_info(a.cu, b, a.T, a.nch, a.B);
    const int c = gc - si.c0;
    if (c < 0 || c >= si.nch) return;  // a slot between two packed sequences' ranges: nothing to prepare
    const int tc0 = c * kC;
    float *sGr = reinterpret_cast<float *>(smem + PrepLds::sGr);

    // g and beta of the chunk for the value heads of this key head (zero past T): requested
    // first, staged in LDS at the end of step 1
    const int ngb = kC * a.r;
    float g_ld[2] = {0.f, 0.f}, b_ld[2] = {0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + 256 * u, row = i / a.r, t = tc0 + row;
        if (i < ngb && t < si.T) {
            const size_t gi = (si.tok0 + t) * a.Hv + kh * a.r + i % a.r;
            g_ld[u] = a.g[gi];
            b_ld[u] = a.beta[gi];
        }
    }
    if (a.A_log) {  // gates from their logits
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + 256 * u, h = kh * a.r + i % a.r;
            if (i < ngb && tc0 + i / a.r < si.T) {
                g_ld[u] = gate_g(g_ld[u], a.A_log[h], a.dt_bias[h]);
                b_ld[u] = gate_beta(b_ld[u]);
            }
        }
    }

    // ---- 1. q/k rows: conv + SiLU + L2 norm.  Thread = (q|k by wave parity, two 4-token
    //         segments, 8 channels)
    {
        const int cg = lane & 15, m = wave & 1;
        const int seg0 = (wave >> 1) * 4 + (lane >> 4);  // segments seg0 and seg0 + 8
        const int ch = m * a.Hk * kD + kh * kD + cg * 8;  // conv channel of element 0
        // rows tc0 - 3 .. tc0 + 63 through one buffer resource from the first row it covers:
        // rows past T read as zero; rows before the sequence come from the conv state
        const int r0 = c > 0 ? tc0 - 3 : 0;
        const unsigned int rowb = (unsigned int)a.Hk * kD * 2;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc((m ? a.k : a.q) + (si.tok0 + r0) * a.Hk * kD + kh * kD,
                      (unsigned int)(min(si.T, tc0 + kC) - r0) * rowb);
        uint4 xr[2][7];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int rr = 0; rr < 7; ++rr) {
                const int t = tc0 + (seg0 + 8 * u) * 4 - 3 + rr;
                xr[u][rr] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rs, (int)((t - r0) * (int)rowb) + cg * 16, 0, 0));
            }
        if (c == 0) {  // the conv-history rows of the first chunk (only segment 0 has any)
#pragma unroll
            for (int rr = 0; rr < 3; ++rr) {
                const int t = seg0 * 4 - 3 + rr;
                if (t < 0)
                    xr[0][rr] = (a.conv && a.conv_state_in)
                                    ? *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + (3 + t)) * a.Cc + ch)
                                    : make_uint4(0, 0, 0, 0);
            }
        }
        // conv taps as bf16 pairs: word 2 e holds taps 0, 1 of channel e, word 2 e + 1 taps 2, 3
        uint4 wr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wr[i] = a.conv ? reinterpret_cast<const uint4 *>(a.conv_w + (size_t)ch * 4)[i] : make_uint4(0, 0, 0, 0);
        const unsigned int wp[16] = {wr[0].x, wr[0].y, wr[0].z, wr[0].w, wr[1].x, wr[1].y, wr[1].z, wr[1].w,
                                     wr[2].x, wr[2].y, wr[2].z, wr[2].w, wr[3].x, wr[3].y, wr[3].z, wr[3].w};
        const float qscale = m ? 1.0f : 0.08838834764831845f;  // 1/sqrt(128) on q
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tl0 = (seg0 + 8 * u) * 4;  // local token of the segment
            float uu[4][8];
            if (a.conv) {
                // The conv as bf16 dot products of tap pairs (the products are exact in fp32):
                // xp[rr][e] pairs channel e of rows rr and rr + 1, so output row i of channel e is
                // dot(taps 0-1, xp[i][e]) + dot(taps 2-3, xp[i + 2][e]).
                unsigned int xw[7][4];
#pragma unroll
                for (int rr = 0; rr < 7; ++rr) {
                    xw[rr][0] = xr[u][rr].x; xw[rr][1] = xr[u][rr].y; xw[rr][2] = xr[u][rr].z; xw[rr][3] = xr[u][rr].w;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        // channels 2 k (low halves) and 2 k + 1 (high halves)
                        const unsigned int lo01 = __builtin_amdgcn_perm(xw[i + 1][k], xw[i][k], 0x05040100u);
                        const unsigned int lo23 = __builtin_amdgcn_perm(xw[i + 3][k], xw[i + 2][k], 0x05040100u);
                        const unsigned int hi01 = __builtin_amdgcn_perm(xw[i + 1][k], xw[i][k], 0x07060302u);
                        const unsigned int hi23 = __builtin_amdgcn_perm(xw[i + 3][k], xw[i + 2][k], 0x07060302u);
                        uu[i][2 * k] = bf16_dot2(wp[4 * k + 1], lo23, bf16_dot2(wp[4 * k], lo01, 0.0f));
                        uu[i][2 * k + 1] = bf16_dot2(wp[4 * k + 3], hi23, bf16_dot2(wp[4 * k + 2], hi01, 0.0f));
                    }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e) uu[i][e] = silu(uu[i][e]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) unpack_bf16x8(xr[u][i + 3], uu[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += uu[i][e] * uu[i][e];
                ss = row16_sum(ss);
                const bool valid = tc0 + tl0 + i < si.T;
                // rows past T are zero; the hardware reciprocal square root (about 1 ulp) is far
                // inside the fp16 the result is stored in
                const float sc = valid ? qscale * __builtin_amdgcn_rsqf(ss + a.eps_l2) : 0.0f;
                half8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = static_cast<_Float16>(uu[i][e] * sc);
                *reinterpret_cast<half8 *>((m ? sK : sQ) + (tl0 + i) * P128 + cg * 8) = hv;
            }
        }
        // raw q/k inputs of the last three tokens -> conv state out
        if (c == 0 && a.conv && a.conv_state_out && tid < 96) {
            const int s = tid >> 5, mm = (tid >> 4) & 1, cq = tid & 15;
            const int tau = si.T - 3 + s;
            const int cc = mm * a.Hk * kD + kh * kD + cq * 8;
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (tau >= 0)
                raw = *reinterpret_cast<const uint4 *>((mm ? a.k : a.q) + ((si.tok0 + tau) * a.Hk + kh) * kD + cq * 8);
            else if (a.conv_state_in)
                raw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + (3 + tau)) * a.Cc + cc);
            *reinterpret_cast<uint4 *>(a.conv_state_out + ((size_t)b * 3 + s) * a.Cc + cc) = raw;
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + 256 * u;
        if (i < ngb) {
            sGr[(i % a.r) * kC + i / a.r] = g_ld[u];
            sGr[(a.r + i % a.r) * kC + i / a.r] = b_ld[u];
        }
    }
    for (int i = tid + 512; i < ngb; i += 256) {  // more than 8 value heads per key head
        const int row = i / a.r, t = tc0 + row;
        const size_t gi = (si.tok0 + t) * a.Hv + kh * a.r + i % a.r;
        const int h = kh * a.r + i % a.r;
        float gv = t < si.T ? a.g[gi] : 0.0f, bv = t < si.T ? a.beta[gi] : 0.0f;
        if (a.A_log && t < si.T) {
            gv = gate_g(gv, a.A_log[h], a.dt_bias[h]);
            bv = gate_beta(bv);
        }
        sGr[(i % a.r) * kC + row] = gv;
        sGr[(a.r + i % a.r) * kC + row] = bv;
    }
    lds_barrier();

    // ---- 1b. q^, k^ and k^T to the workspace as operand fragments
    {
        // Wave w writes fragments w + 4 it: q^ for it < 4, k^ for it >= 4, each at row tile it & 3
        // and key step w, so every source address is the lane's base plus a constant.
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.qkf + ((size_t)gc * a.Hk + kh) * kQKF, kQKF * 2);
        const int fl = lane & 15, fq = lane >> 4;
        {
            const int lb = fl * P128 + 32 * wave + 4 * fq;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const _Float16 *src = (it < 4 ? sQ : sK) + lb + 16 * (it & 3) * P128;
                const half4 lo = lds_half4(src), hi = lds_half4(src + 16);
                st_ws(rq, (tid + 256 * it) * 16, half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
            }
        }
        // k^T fragment 32 + 2 ti + s2, lane fl + 16 fq: key 16 ti + fl at tokens
        // 32 s2 + 4 fq + e and 32 s2 + 16 + 4 fq + e (e = 0..3).  Wave w writes fragments
        // 32 + w + 4 it: s2 = w & 1, ti = (w >> 1) + 2 it.
        {
            const _Float16 *lb = sK + (32 * (wave & 1) + 4 * fq) * P128 + 16 * (wave >> 1) + fl;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const _Float16 *src = lb + 32 * it;
                half8 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = src[e * P128];
                    v[4 + e] = src[(16 + e) * P128];
                }
                st_ws(rq, (32 * 64 + tid + 256 * it) * 16, v);
            }
        }
    }

    // ---- 2. cumulative log-decays of every value head (wave w takes heads w, w + 4, ...) and
    //         their decay vectors to the workspace; then the raw K K^T tiles of L and the
    //         K Q^T tiles of P, kept in registers
    for (int hr = wave; hr < a.r; hr += 4) {
        const __amdgpu_buffer_rsrc_t rtp = make_rsrc(a.tpf + ((size_t)gc * a.Hv + kh * a.r + hr) * kTPF, kTPF * 2);
        float gv = sGr[hr * kC + lane];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float t2 = __shfl_up(gv, o, 64);
            if (lane >= o) gv += t2;
        }
        const float gC = __shfl(gv, 63, 64);
        sGr[hr * kC + lane] = gv;
        st_ws(rtp, kVecOff * 2 + 4 * lane, hw_exp(gv));
        st_ws(rtp, kVecOff * 2 + 4 * (kC + lane), hw_exp(gC - gv));
        if (lane < 4) st_ws(rtp, kVecOff * 2 + 4 * (2 * kC + lane), hw_exp(gC));
    }
    // P fragments: operand fragment f of P (row block fI, token step fks) is built from the
    // K Q^T tiles (fI, 2 fks) and (fI, 2 fks + 1): with K as the A operand and Q as the B operand
    // the accumulator lane holds query row i = 16 fI + l16 at keys j = 16 J + 4 lq + e, which is
    // the fragment's own lane layout, so P needs no staging.  Tiles above the diagonal are zero.
    // Wave w owns fragments kPF[w] (6 fragments, 10 nonzero tiles over the four waves).  The
    // K K^T tile of L for the same (i, j) block comes from the same A operand with K as the B
    // operand (K K^T is symmetric), so the lane holding P_ij also holds the raw L_ij and one
    // exponential e^{G_i - G_j} serves both.
    constexpr int kPF[4][2] = {{1, 0}, {3, 2}, {4, -1}, {5, -1}};
    constexpr int kFI[6] = {0, 1, 2, 2, 3, 3}, kFKS[6] = {0, 0, 0, 1, 0, 1};
    floatx4 rawP[2][2], rawL[2][2];
#pragma unroll
    for (int pf = 0; pf < 2; ++pf) {
        const int f = kPF[wave][pf];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            rawP[pf][hh] = rawL[pf][hh] = floatx4{0.f, 0.f, 0.f, 0.f};
            const int J = f >= 0 ? 2 * kFKS[f] + hh : 0, fI = f >= 0 ? kFI[f] : 0;
            if (f >= 0 && J <= fI) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const half8 av = lds_half8(sK + (16 * J + l16) * P128 + 32 * ks + 8 * lq);
                    const half8 bq = lds_half8(sQ + (16 * fI + l16) * P128 + 32 * ks + 8 * lq);
                    const half8 bk = lds_half8(sK + (16 * fI + l16) * P128 + 32 * ks + 8 * lq);
                    rawP[pf][hh] = mfma16x16x32(av, bq, rawP[pf][hh]);
                    rawL[pf][hh] = mfma16x16x32(av, bk, rawL[pf][hh]);
                }
            }
        }
    }
    lds_barrier();

    // ---- 3. per value head of this key head
    for (int hr = 0; hr < a.r; ++hr) {
        const int h = kh * a.r + hr;
        const __amdgpu_buffer_rsrc_t rtp = make_rsrc(a.tpf + ((size_t)gc * a.Hv + h) * kTPF, kTPF * 2);
        const float *sG = sGr + hr * kC;          // cumulative log-decay G
        const float *sB = sGr + (a.r + hr) * kC;  // beta

        // P = (Q K^T) o R (lower incl. the diagonal), straight from registers to the workspace, and
        // L = strictly-lower(beta_i (K K^T) o R) (fp32) to LDS rows, from the same exponentials
#pragma unroll
        for (int pf = 0; pf < 2; ++pf) {
            const int f = kPF[wave][pf];
            if (f < 0) continue;
            const int fI = kFI[f], i = 16 * fI + l16;
            const float gi = sG[i], bi = sB[i];
            half8 v;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int J = 2 * kFKS[f] + hh, j0 = 16 * J + 4 * lq;
                if (J > fI) {  // above the diagonal (uniform): P is zero, L is never read
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[4 * hh + e] = static_cast<_Float16>(0.0f);
                    continue;
                }
                const float4 gj = *reinterpret_cast<const float4 *>(sG + j0);
                const float gjs[4] = {gj.x, gj.y, gj.z, gj.w};
                float lv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ex = hw_exp(gi - gjs[e]);
                    v[4 * hh + e] = static_cast<_Float16>(keep_if_nonneg(i - (j0 + e), rawP[pf][hh][e] * ex));
                    lv[e] = keep_if_nonneg(i - (j0 + e) - 1, bi * rawL[pf][hh][e] * ex);
                }
                *reinterpret_cast<float4 *>(sL + i * PL + j0) = make_float4(lv[0], lv[1], lv[2], lv[3]);
            }
            st_ws(rtp, (kPOff + f * kFrag) * 2 + lane * 16, v);
        }
        lds_barrier();

        // diagonal 16x16 blocks of T = (I + L)^{-1}: forward substitution, one column per lane,
        // column-oriented (once x[mm] is final it is subtracted from every later row at once),
        // so the dependent steps are the 15 rows rather than every product; the products and
        // their order per row are those of the row-by-row form.  One wave takes all four
        // blocks (block lane / 16, column lane % 16): the same dependent steps with every lane
        // busy, where one block per wave left three quarters of four waves' issue slots idle
        // (this kernel is bound by VALU issue)
        if (wave == (hr & 3)) {
            const int blk = lane >> 4, w0 = 16 * blk, cidx = lane & 15;
            float x[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) x[rr] = rr == cidx ? 1.0f : 0.0f;
#pragma unroll
            for (int mm = 0; mm < 15; ++mm) {
                const float xm = x[mm];
#pragma unroll
                for (int rr = mm + 1; rr < 16; ++rr) x[rr] -= sL[(w0 + rr) * PL + w0 + mm] * xm;
            }
            const float bc = sB[w0 + cidx];
            const int db = blk * (blk + 1) / 2 + blk;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                sTd[(blk * 16 + rr) * PTD + cidx] = x[rr];
                sT16T[(w0 + cidx) * P64 + w0 + rr] = static_cast<_Float16>(x[rr]);
                sTbst[db * kBlk + rr * kTBS + cidx] = static_cast<_Float16>(x[rr] * bc);
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
                    // one 16-byte read per lane (four 4-byte reads of it put two lanes on a bank)
                    const float4 l4 = *reinterpret_cast<const float4 *>(sL + (16 * I + l16) * PL + 16 * K + 4 * lq);
                    const half4 av = {static_cast<_Float16>(l4.x), static_cast<_Float16>(l4.y),
                                      static_cast<_Float16>(l4.z), static_cast<_Float16>(l4.w)};
                    const half4 bv = lds_half4(sT16T + (16 * J + l16) * P64 + 16 * K + 4 * lq);
                    y = mfma16x16x16(av, bv, y);
                }
                // y's accumulator layout is the B-operand layout of the next product
                half4 yb;
#pragma unroll
                for (int e = 0; e < 4; ++e) yb[e] = static_cast<_Float16>(y[e]);
                const float4 t4 = *reinterpret_cast<const float4 *>(sTd + (I * 16 + l16) * PTD + 4 * lq);
                const half4 tv = {static_cast<_Float16>(t4.x), static_cast<_Float16>(t4.y),
                                  static_cast<_Float16>(t4.z), static_cast<_Float16>(t4.w)};
                floatx4 t = {0.f, 0.f, 0.f, 0.f};
                t = mfma16x16x16(tv, yb, t);
                half4 th;
                const int blk = I * (I + 1) / 2 + J;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    th[e] = static_cast<_Float16>(-t[e]);
                    sTbst[blk * kBlk + (4 * lq + e) * kTBS + l16] = static_cast<_Float16>(-t[e] * bcol);
                }
                *reinterpret_cast<half4 *>(sT16T + (16 * J + l16) * P64 + 16 * I + 4 * lq) = th;
                wave_lds_sync();
            }
        }
        lds_barrier();

        // T diag(beta) to the workspace as fragments 0..5: row tiles 0 and 1 take the first token
        // step only, row tiles 2 and 3 both
        // (wave w writes fragments w and w + 4; the row block bi and token step ks are uniform)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int f = wave + 4 * it;
            if (f >= 6) break;
            const int fl = lane & 15, fq = lane >> 4;
            const int bi = f < 2 ? f : 2 + ((f - 2) >> 1);
            const int ks = f < 2 ? 0 : (f - 2) & 1;
            half8 v;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int bj = 2 * ks + hh;  // the 16-column block of these 4 columns
                half4 q4 = {0, 0, 0, 0};
                if (bj <= bi) q4 = lds_half4(sTbst + (bi * (bi + 1) / 2 + bj) * kBlk + fl * kTBS + 4 * fq);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * hh + e] = q4[e];
            }
            st_ws(rtp, (f * 64 + lane) * 16, v);
        }
        // (no barrier: the next head writes T staging only after its own first barrier, which
        // every wave reaches after finishing these reads)
    }
}

// ========================================================================
// segment_pass_kernel: the first pass of the two-level scan
// ========================================================================
//
// Every segment of seg_chunks chunks runs on its own, with 256 virtual value columns per
// head: columns 0..127 start from the identity and carry no values (their state ends as
// the segment's transition M, their read-out as R, so that R S_start is what the start
// state adds to the outputs), columns 128..255 start from zero with the real values
// (state N, read-out O0).  A segment's outputs are then O0 + R S_start and its final state
// M S_start + N (the segment map is affine in the start state), which the two later
// kernels apply.  One workgroup of 8 waves per (sequence, value head, segment, slice of
// 32 virtual columns).  Pipeline of one iteration c (every role runs iterations
// 0..nch+2+kSegLag with one LDS barrier each; the lags keep every hand-off one barrier or
// more away):
//   A (state, waves 0, 1)     chunk c: X, Delta, S update; Sb(c), Db(c) -> LDS
//   B (read-out, waves 2, 3)  chunk c-1: O = e^G Q S + P Delta -> sO
//   L (load, wave 5)          DMA of the k^ fragments of chunk c+2 and the raw v of chunk
//                             c+3; a DMA issued in iteration c is complete at the barrier
//                             that ends iteration c+1, so its data is used from c+2 on
//   V (helpers, waves 4, 6, 7) conv + SiLU of v for chunk c+1; the read-out of chunk
//                             c-3-kSegLag to the workspace in fp16
constexpr int kSegLag = 3;
constexpr int kORing = kSegLag + 3;  // read-out tiles in LDS
constexpr int kSegNT = 2;            // 16-column tiles per workgroup
constexpr int kOpSlot = 16 * 1024;   // operand slot: the chunk's k^ fragments
constexpr int kSD = 6 * 1024;        // per tile: Sb (4 fragments) and Db (2 fragments)

struct SegPassArgs {
    const _Float16 *qkf, *tpf;
    const uint16_t *v, *conv_w, *conv_state_in;
    uint16_t *conv_state_out;
    unsigned int *tickets;     // [8] next item of each XCD queue
    unsigned int *exits;       // workgroups that have left the item loop
    _Float16 *seg_out;         // per (chunk slot, value head) kSegBlk halves: R as MFMA A fragments, O0 rows
    float *seg_state;          // [B Hv nseg][128][256] fp32: final [M | N] of each segment
    int nseg, seg_chunks;
    int B, T, Hk, Hv, r, Cc, conv, nch, n_items, grid;
};

template <int NT>
struct ChainLds {
    static constexpr int BV = 16 * NT;
    static constexpr int VT = BV * PL;                          // floats of one column-major [BV][64] tile
    static constexpr int NSLOT = 3;                              // ring depth of the DMA'd operands and raw v
    static constexpr size_t sOp = 0;                             // [NSLOT][kOpSlot]     DMA'd operands
    static constexpr size_t sSD = sOp + (size_t)NSLOT * kOpSlot; // [2][NT][kSD]         Sb, Db fragments per tile
    static constexpr size_t sV = sSD + 2 * NT * kSD;             // fp16 [2][BV][P64]     conv(v) of the slice
    static constexpr size_t sO = sV + 2 * 2 * BV * P64;          // fp32 [kORing][BV][PL] read-out
    static constexpr size_t sRawV = sO + 4 * kORing * VT;        // bf16 [NSLOT][64][BV]  raw v
    static constexpr size_t sHalo = sRawV + 2 * NSLOT * kC * BV; // bf16 [2][3][BV]       raw v rows before a chunk
    static constexpr size_t sCW = sHalo + 2 * 2 * 3 * BV;        // fp32 [BV][4]          conv taps of the v channels
    static constexpr size_t bytes = sCW + 4 * 4 * BV;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Position in LDS of the 16-byte piece of k^ fragment lane L = 16 b + 4 c + a:
// 16 b + 4 (c ^ b) + a (an involution).  The transposing reads of the state update
// take, per 16-lane group, the pieces of lanes 4 c + a + 16 b for one c; stored in
// lane order those pieces fall on only four bank groups, swizzled on sixteen, and
// the plain 16-lane phases of the operand reads stay conflict-free as well.
__device__ __forceinline__ int kswz(int L) { return (L & 0x33) | ((((L >> 2) ^ (L >> 4)) & 3) << 2); }

// Operands of one chunk that the state wave keeps in registers (loaded one
// chunk ahead): T diag(beta) fragments and the decay vectors.
struct StateFrags {
    half8 tb[6];
    float4 eg[4], egc[4];  // e^{G}, e^{G_C - G}: rows 16 I + 4 lq .. +3
    float dC;              // e^{G_C}
};

__device__ __forceinline__ void state_load(StateFrags &fr, const _Float16 *tpb, int lane, int lq) {
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(tpb, kTPF * 2);
#pragma unroll
    for (int f = 0; f < 6; ++f) fr.tb[f] = ld_frag(rt, lane * 16, f);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        fr.eg[u] = ld_f4(rt, kVecOff * 2 + lq * 16, 64 * u);
        fr.egc[u] = ld_f4(rt, kVecOff * 2 + lq * 16, 256 + 64 * u);
    }
    fr.dC = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rt, 0, kVecOff * 2 + 4 * 2 * kC, 0));
}

// One chunk of the state chain for one 16-column tile (an A wave):
// X = V - e^G (K S); Delta = T diag(beta) X; S = e^{G_C} S + K^T (e^{G_C - G} Delta).
// S holds the tile in the accumulator layout (key-row tiles ti = 0..7); k^
// fragments come from LDS (k^T through the transposing read); Sb (S before the
// chunk) and Db (Delta) go to LDS for the output wave of the tile.  fr is
// reloaded with the next chunk's (tpn) operands after its last use.
template <int NT>
__device__ __forceinline__ void state_step(unsigned char *smem, floatx4 (&S)[8], StateFrags &fr,
                                           const _Float16 *tpn, int c, int t, int lane, int jc, int lq, int trofs) {
    using L = ChainLds<NT>;
    const unsigned char *op = smem + L::sOp + (c % L::NSLOT) * kOpSlot;
    const _Float16 *opk = reinterpret_cast<const _Float16 *>(op);
    const _Float16 *sVc = reinterpret_cast<const _Float16 *>(smem + L::sV) + (c & 1) * L::BV * P64;
    half8 *sd = reinterpret_cast<half8 *>(smem + L::sSD + ((c & 1) * NT + t) * kSD) + lane;

    half8 fk[16];
#pragma unroll
    for (int f = 0; f < 16; ++f) fk[f] = *reinterpret_cast<const half8 *>(op + f * 1024 + kswz(lane) * 16);
    half4 vv[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) vv[I] = lds_half4(sVc + jc * P64 + 16 * I + 4 * lq);
    half8 Sb[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        Sb[s2] = pack_tiles(S[2 * s2], S[2 * s2 + 1]);
        sd[64 * s2] = Sb[s2];
    }
    __builtin_amdgcn_sched_barrier(0);

    // K S (k-step outermost: four accumulation chains in flight), X = V - e^G K S
    floatx4 ks[4] = {};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int I = 0; I < 4; ++I) ks[I] = mfma16x16x32(fk[4 * I + s2], Sb[s2], ks[I]);
    floatx4 X[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        X[I][0] = (float)vv[I][0] - fr.eg[I].x * ks[I][0];
        X[I][1] = (float)vv[I][1] - fr.eg[I].y * ks[I][1];
        X[I][2] = (float)vv[I][2] - fr.eg[I].z * ks[I][2];
        X[I][3] = (float)vv[I][3] - fr.eg[I].w * ks[I][3];
    }
    const half8 Xb[2] = {pack_tiles(X[0], X[1]), pack_tiles(X[2], X[3])};

    // Delta = T diag(beta) X  (lower triangular: 32-row block s2 uses k-steps <= s2)
    half8 Dsb[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
        if (s2 == 0) {
            d0 = mfma16x16x32(fr.tb[0], Xb[0], d0);
            d1 = mfma16x16x32(fr.tb[1], Xb[0], d1);
        } else {
            d0 = mfma16x16x32(fr.tb[2], Xb[0], d0);
            d0 = mfma16x16x32(fr.tb[3], Xb[1], d0);
            d1 = mfma16x16x32(fr.tb[4], Xb[0], d1);
            d1 = mfma16x16x32(fr.tb[5], Xb[1], d1);
        }
        sd[64 * (4 + s2)] = pack_tiles(d0, d1);
        const float4 c0 = fr.egc[2 * s2], c1 = fr.egc[2 * s2 + 1];
        Dsb[s2] = half8{(_Float16)(d0[0] * c0.x), (_Float16)(d0[1] * c0.y), (_Float16)(d0[2] * c0.z),
                        (_Float16)(d0[3] * c0.w), (_Float16)(d1[0] * c1.x), (_Float16)(d1[1] * c1.y),
                        (_Float16)(d1[2] * c1.z), (_Float16)(d1[3] * c1.w)};
    }
#pragma unroll
    for (int ti = 0; ti < 8; ++ti) S[ti] = S[ti] * fr.dC;
    __builtin_amdgcn_sched_barrier(0);
    state_load(fr, tpn, lane, lq);

    // S += K^T Delta~: k^T fragments from the k^ fragments through the transposing read
    // (tokens 32 s2 + {4 lq + j}: k^ fragment 8 s2 + (ti >> 1); tokens +16: 4 fragments on;
    // the keys of tile ti are the 8-byte half (ti & 1) of each lane's 16 bytes)
#pragma unroll
    for (int ti = 0; ti < 8; ++ti) {
        floatx4 acc = S[ti];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const _Float16 *base = opk + (8 * s2 + (ti >> 1)) * kFrag + 4 * (ti & 1) + trofs;
            const half4 lo = lds_tr16(base), hi = lds_tr16(base + 4 * kFrag);
            acc = mfma16x16x32(half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, Dsb[s2], acc);
        }
        S[ti] = acc;
    }
}

// Read-out of one chunk for one 16-column tile (a B wave): O = e^G (Q S) + P Delta
// with Sb, Db from the A wave of the tile; O to LDS (column-major).
struct OutFrags {
    half8 q[16], p[6];
    float4 eg[4];
};

__device__ __forceinline__ void out_load(OutFrags &fr, const _Float16 *qkb, const _Float16 *tpb, int lane, int lq) {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qkb, kQKF * 2), rt = make_rsrc(tpb, kTPF * 2);
#pragma unroll
    for (int f = 0; f < 16; ++f) fr.q[f] = ld_frag(rq, lane * 16, f);
#pragma unroll
    for (int f = 0; f < 6; ++f) fr.p[f] = ld_frag(rt, kPOff * 2 + lane * 16, f);
#pragma unroll
    for (int u = 0; u < 4; ++u) fr.eg[u] = ld_f4(rt, kVecOff * 2 + lq * 16, 64 * u);
}

template <int NT>
__device__ __forceinline__ void out_step(unsigned char *smem, const OutFrags &fr, int c, int t, int lane, int jc,
                                         int lq) {
    using L = ChainLds<NT>;
    const half8 *sd = reinterpret_cast<const half8 *>(smem + L::sSD + ((c & 1) * NT + t) * kSD) + lane;
    float *sOc = reinterpret_cast<float *>(smem + L::sO) + (c % kORing) * L::VT;
    half8 Sb[4], Db[2];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) Sb[s2] = sd[64 * s2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) Db[s2] = sd[64 * (4 + s2)];
    floatx4 qs[4] = {};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int I = 0; I < 4; ++I) qs[I] = mfma16x16x32(fr.q[4 * I + s2], Sb[s2], qs[I]);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        floatx4 ot = {qs[I][0] * fr.eg[I].x, qs[I][1] * fr.eg[I].y, qs[I][2] * fr.eg[I].z, qs[I][3] * fr.eg[I].w};
        if (I < 2) {
            ot = mfma16x16x32(fr.p[I], Db[0], ot);
        } else {
            ot = mfma16x16x32(fr.p[2 + 2 * (I - 2)], Db[0], ot);
            ot = mfma16x16x32(fr.p[3 + 2 * (I - 2)], Db[1], ot);
        }
        *reinterpret_cast<float4 *>(sOc + jc * PL + 16 * I + 4 * lq) = make_float4(ot[0], ot[1], ot[2], ot[3]);
    }
}



// Two-level scan: what the first pass hands the last one per (chunk slot, value head), in fp16:
// R [64][128] (the read-out of the transition columns) as 16 MFMA A-operand fragments
// (row tile rt, k-step ks: lane l16 + 16 lq holds row 16 rt + l16 at columns 32 ks + 4 lq + e
// and 32 ks + 16 + 4 lq + e), then O0 [64][128] (the zero-start read-out) row-major.
constexpr int kSegR = 16 * kFrag;
constexpr int kSegBlk = kSegR + kC * kD;

// grid: min(items, resident slots), 512 threads
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void segment_pass_kernel(SegPassArgs a) {
    constexpr int NT = kSegNT;
    using L = ChainLds<NT>;
    constexpr int BV = L::BV, VT = L::VT;
    constexpr int NSL = 2 * kTiles / NT;        // slices of the 256 virtual columns
    constexpr int NCG = BV / 8;                 // 8-column groups per slice row
    // Helpers 0..2 (waves 4, 6, 7).  The conv of rows 0..31 goes to helper 0 and of rows
    // 32..63 to helper 1; the read-out's 256 row pieces go to helper 1 (64) and helper 2 (192).
    constexpr int kOutLanes = 128;              // helper lanes 64..191
    constexpr int kConvLanes = 128;             // helper lanes 0..127
    constexpr int NRD = kC * BV * 2 / 1024;     // DMA instructions for 64 rows of raw v of the slice
    constexpr int GROUP = kOpSlot / 1024 + NRD; // DMA instructions the load wave issues per iteration
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    _Float16 *sV = reinterpret_cast<_Float16 *>(smem + L::sV);
    float *sO = reinterpret_cast<float *>(smem + L::sO);
    uint16_t *sRawV = reinterpret_cast<uint16_t *>(smem + L::sRawV);
    uint16_t *sHalo = reinterpret_cast<uint16_t *>(smem + L::sHalo);
    float *sCW = reinterpret_cast<float *>(smem + L::sCW);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: role branches are scalar
    const int l16 = lane & 15, lq = lane >> 4;
    // Waves w and w + 4 share a SIMD: the state waves (0, 1) are paired with the lightest
    // roles, helper 0 (conv only) at 4 and the load wave at 5.
    constexpr int kLoadWave = 5;
    const bool is_a = wave < NT, is_b = wave >= NT && wave < 2 * NT, is_l = wave == kLoadWave;
    const int vh = wave == 4 ? 0 : wave - 5;    // helper index of waves 4, 6, 7
    __shared__ int s_item;
    // Work items (segment chain, slice) come from eight queues, one per XCD: chain c sits
    // in queue c % 8 and its slices are consecutive tickets.  A workgroup serves the queue
    // of the XCD it runs on (the slices of a chain then share that XCD's L2), and the other
    // queues once its own is empty.  No workgroup ever waits for another one.
    const int xcc = static_cast<int>(xcc_id() & 7u);
    const int n_chains = a.B * a.Hv * a.nseg;  // (head, segment) pairs
    int qi = 0;

    for (;;) {
        if (tid == 0) {
            auto queue_len = [&](int q) { return (unsigned int)((n_chains > q ? (n_chains - q + 7) / 8 : 0) * NSL); };
            int item = -1;
            while (qi < 8 && item < 0) {
                const int q = (xcc + qi) & 7;
                const unsigned int tk = __hip_atomic_fetch_add(a.tickets + q, 1u, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT);
                if (tk < queue_len(q)) {
                    item = (q + 8 * (int)(tk / NSL)) * NSL + (int)(tk % NSL);
                } else {
                    // queue q is used up (tickets only grow during a launch): read every queue's
                    // count at once, one memory latency, and skip to the first that still has
                    // items, if any, instead of trying the queues one atomic at a time
                    unsigned int seen[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        seen[j] = __hip_atomic_load(a.tickets + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ++qi;
                    while (qi < 8 && seen[(xcc + qi) & 7] >= queue_len((xcc + qi) & 7)) ++qi;
                }
            }
            s_item = item;
        }
        __syncthreads();
        const int item = __builtin_amdgcn_readfirstlane(s_item);  // uniform: addresses stay scalar
        __syncthreads();
        if (item < 0) break;
        const int vchain = item / NSL, s = item % NSL;
        const int chain = vchain / a.nseg, seg = vchain % a.nseg;
        const int b = chain / a.Hv, h = chain % a.Hv, kh = h / a.r;
        const SeqInfo si = seq_info(nullptr, b, a.T, a.nch, a.B);  // the whole sequence (an even batch)
        SeqInfo ss = si;                                             // the segment
        {
            const int cb = seg * a.seg_chunks;
            ss.tok0 = si.tok0 + (size_t)cb * kC;
            ss.T = min(si.T - cb * kC, a.seg_chunks * kC);
            ss.c0 = si.c0 + cb;
            ss.nch = min(si.nch - cb, a.seg_chunks);
        }
        const int nch = ss.nch, sc0 = ss.c0;      // at least one chunk: the plan leaves no segment empty
        const int vcol0 = s * BV;                 // virtual column 0..255
        const bool mcol = vcol0 < kD;             // transition columns: identity start, no values
        const int sv0 = vcol0 % kD;               // value column of the slice
        const int last = nch + 2 + kSegLag;
        const size_t qk_stride = (size_t)a.Hk * kQKF, tp_stride = (size_t)a.Hv * kTPF;
        const _Float16 *qk0 = a.qkf + ((size_t)sc0 * a.Hk + kh) * kQKF;
        const _Float16 *tp0 = a.tpf + ((size_t)sc0 * a.Hv + h) * kTPF;

        if (is_a) {
            // ---------------------------------------------------------- state wave
            const int jc = 16 * wave + l16;
            // transposing-read lane offset (fp16 elements): row j = l16 / 4 of the 16-lane
            // group, 4-key chunk q = l16 % 4 -> k^ fragment lane (4 lq + j) + 16 q, at its
            // swizzled LDS position
            const int trofs = kswz((4 * lq + (l16 >> 2)) + 16 * (l16 & 3)) * 8;
            StateFrags fr;
            state_load(fr, tp0, lane, lq);
            floatx4 S[8];
#pragma unroll
            for (int ti = 0; ti < 8; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[ti][e] = (mcol && 16 * ti + 4 * lq + e == sv0 + jc) ? 1.0f : 0.0f;
            lds_barrier();
            lds_barrier();
            for (int c = 0; c <= last; ++c) {
                if (c < nch)
                    state_step<NT>(smem, S, fr, tp0 + min(c + 1, nch - 1) * tp_stride, c, wave, lane, jc, lq, trofs);
                lds_barrier();
            }
#pragma unroll
            for (int ti = 0; ti < 8; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.seg_state[((size_t)vchain * kD + 16 * ti + 4 * lq + e) * (2 * kD) + vcol0 + jc] = S[ti][e];
        } else if (is_b) {
            // ---------------------------------------------------------- read-out wave
            const int t = wave - NT, jc = 16 * t + l16;
            OutFrags fr;
            out_load(fr, qk0, tp0, lane, lq);
            lds_barrier();
            lds_barrier();
            for (int c = 0; c <= last; ++c) {
                if (c >= 1 && c - 1 < nch) {
                    out_step<NT>(smem, fr, c - 1, t, lane, jc, lq);
                    if (c < nch) out_load(fr, qk0 + c * qk_stride, tp0 + c * tp_stride, lane, lq);
                }
                lds_barrier();
            }
        } else if (is_l) {
            // ---------------------------------------------------------- load wave (DMA only)
            // raw v rows of chunk cc: a buffer from the chunk's first token, so rows past T read as 0;
            // lane -> row (64 / NRD rows per instruction), 8-column group
            auto rows_dma = [&](int cc, uint16_t *dst) __attribute__((always_inline)) {
                const int c0 = min(max(cc, 0), nch - 1) * kC;
                const unsigned int nrow = (unsigned int)min(ss.T - c0, kC);
                const __amdgpu_buffer_rsrc_t r =
                    make_rsrc(a.v + (ss.tok0 + c0) * a.Hv * kD, nrow * (unsigned int)a.Hv * kD * 2);
#pragma unroll
                for (int u = 0; u < NRD; ++u) {
                    const int i = lane + 64 * u, row = i / NCG, cg = i % NCG;
                    dma16b(r, ((row * a.Hv + h) * kD + sv0 + 8 * cg) * 2, dst + u * 512);
                }
            };
            auto ops_dma = [&](int cc) __attribute__((always_inline)) {
                const int cl = min(cc, nch - 1);  // (past the last chunk: a harmless duplicate)
                unsigned char *slot = smem + L::sOp + (cc % L::NSLOT) * kOpSlot;
                const _Float16 *kb = qk0 + cl * qk_stride + kKOff;
#pragma unroll
                for (int f = 0; f < 16; ++f) dma16(kb + f * kFrag + kswz(lane) * 8, slot + f * 1024);
            };
            // prologue: operands of chunks 0 and 1, raw v of chunks 0..2
            ops_dma(0);
            ops_dma(1);
#pragma unroll
            for (int j = 0; j <= 2; ++j) rows_dma(j, sRawV + j * kC * BV);
            wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_s_barrier();
            for (int c = 0; c <= last; ++c) {
                // this iteration's group (the same instructions in every iteration, past the last
                // chunk from the last chunk's rows, so that the count below is exact): operands of
                // chunk c+2, raw v of chunk c+3
                ops_dma(c + 2);
                rows_dma(c + 3, sRawV + ((c + 3) % L::NSLOT) * kC * BV);
                // the group of iteration c has landed; this one may still be in flight
                wait_vmcnt<GROUP>();
                __builtin_amdgcn_s_barrier();
            }
            wait_vmcnt<0>();
        } else {
            // ---------------------------------------------------------- VALU helpers
            const int vtid = vh * 64 + lane;
            if (vtid < BV) {
                const int chn = 2 * a.Hk * kD + h * kD + sv0 + vtid;
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4)
                    sCW[vtid * 4 + t4] = a.conv ? bf16_to_f32(a.conv_w[(size_t)chn * 4 + t4]) : 0.0f;
            }
            // the three raw rows before the segment: the conv state in (or zeros) for the
            // first segment, the sequence's own rows for a later one
            if (vtid >= 64 && vtid < 64 + 3 * NCG) {
                const int r3 = (vtid - 64) / NCG, cg = (vtid - 64) % NCG;
                uint4 rw = make_uint4(0, 0, 0, 0);
                if (a.conv && !mcol) {
                    if (seg > 0)
                        rw = *reinterpret_cast<const uint4 *>(a.v + ((ss.tok0 - 3 + r3) * a.Hv + h) * kD + sv0 + cg * 8);
                    else if (a.conv_state_in)
                        rw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + r3) * a.Cc +
                                                              2 * a.Hk * kD + h * kD + sv0 + cg * 8);
                }
                *reinterpret_cast<uint4 *>(sHalo + r3 * BV + cg * 8) = rw;
            }
            const int cgl = vtid % NCG;  // a lane always serves the same 8-column group
            // conv + SiLU of v for chunk cc (its raw rows from the ring, the three rows before it
            // from sHalo[cc & 1]) -> sV[cc & 1]; the chunk's last three raw rows -> sHalo[(cc + 1) & 1].
            // Conv lane ci owns RPI = 4 consecutive rows of 4 channels: it reads each raw row it
            // needs once (RPI + 3 rows of 8 bytes) and writes each channel's RPI outputs as one
            // packed store.
            constexpr int RPI = 4;
            constexpr int NC4 = BV / 4;
            static_assert((kC / RPI) * NC4 == kConvLanes, "one conv item per conv lane");
            const int ci = vtid < kConvLanes ? vtid : -1;  // conv lane
            const int c4 = (ci > 0 ? ci : 0) % NC4, rg = (ci > 0 ? ci : 0) / NC4;
            float hwc[16];  // conv taps of the lane's 4 channels: tap j of channel e at 4 e + j
            auto conv_v = [&](int cc) __attribute__((always_inline)) {
                if (ci < 0) return;  // not a converting helper
                const uint16_t *raw = sRawV + (cc % L::NSLOT) * kC * BV;
                if (ci < 3 * NCG) {
                    const int r3 = ci / NCG, cg = ci % NCG;
                    *reinterpret_cast<uint4 *>(sHalo + ((cc + 1) & 1) * 3 * BV + r3 * BV + cg * 8) =
                        *reinterpret_cast<const uint4 *>(raw + (kC - 3 + r3) * BV + cg * 8);
                }
                const int r0 = rg * RPI;
                uint2 rw[RPI + 3];
#pragma unroll
                for (int j = 0; j < RPI + 3; ++j) {
                    const int r2 = r0 - 3 + j;  // rows before the chunk come from the halo
                    rw[j] = *reinterpret_cast<const uint2 *>(
                        r2 >= 0 ? raw + r2 * BV + c4 * 4 : sHalo + (cc & 1) * 3 * BV + (3 + r2) * BV + c4 * 4);
                }
                __builtin_amdgcn_sched_barrier(0);
                float x[RPI + 3][4];
#pragma unroll
                for (int j = 0; j < RPI + 3; ++j) {
                    x[j][0] = __uint_as_float(rw[j].x << 16);
                    x[j][1] = __uint_as_float(rw[j].x & 0xffff0000u);
                    x[j][2] = __uint_as_float(rw[j].y << 16);
                    x[j][3] = __uint_as_float(rw[j].y & 0xffff0000u);
                }
                float u[RPI][4];
#pragma unroll
                for (int i = 0; i < RPI; ++i) {
                    if (mcol) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) u[i][e] = 0.0f;
                    } else if (a.conv) {
                        float acc[4], t4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[e] = hwc[4 * e] * x[i][e] + hwc[4 * e + 1] * x[i + 1][e] + hwc[4 * e + 2] * x[i + 2][e] +
                                     hwc[4 * e + 3] * x[i + 3][e];
#pragma unroll
                        for (int e = 0; e < 4; ++e) t4[e] = __builtin_amdgcn_exp2f(acc[e] * -1.4426950408889634f);
#pragma unroll
                        for (int e = 0; e < 4; ++e) t4[e] = __builtin_amdgcn_rcpf(1.0f + t4[e]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) u[i][e] = acc[e] * t4[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) u[i][e] = x[i + 3][e];
                    }
                }
                _Float16 *dst = sV + (cc & 1) * BV * P64 + c4 * 4 * P64 + r0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<half4 *>(dst + e * P64) =
                        half4{static_cast<_Float16>(u[0][e]), static_cast<_Float16>(u[1][e]),
                              static_cast<_Float16>(u[2][e]), static_cast<_Float16>(u[3][e])};
            };
            // the raw read-out of chunk oc to the workspace for the last kernel (every row: rows
            // past T are finite): R as two 4-column pieces of one row in two lanes of a fragment,
            // O0 as 8 columns of one row
            auto emit = [&](int oc) __attribute__((always_inline)) {
                const float *src = sO + (oc % kORing) * VT + cgl * 8 * PL;
                _Float16 *blk = a.seg_out + ((size_t)(sc0 + oc) * a.Hv + h) * kSegBlk;
                const int col = sv0 + cgl * 8;
                const int gstep = vh == 1 ? kC * NCG : 64;  // helper 1 one row piece per lane, helper 2 three
#pragma unroll 1
                for (int it = vtid - 64; it < kC * NCG; it += gstep) {
                    const int row = it / NCG;
                    float y[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] = src[e * PL + row];
                    if (mcol) {
                        const int cc = col & 31, L0 = (row & 15) + 16 * ((cc & 15) >> 2);
                        _Float16 *f = blk + (((row >> 4) * 4 + (col >> 5)) * 64 + L0) * 8 + 4 * (cc >> 4);
                        *reinterpret_cast<half4 *>(f) = half4{(_Float16)y[0], (_Float16)y[1], (_Float16)y[2],
                                                              (_Float16)y[3]};
                        *reinterpret_cast<half4 *>(f + 16 * 8) = half4{(_Float16)y[4], (_Float16)y[5],
                                                                       (_Float16)y[6], (_Float16)y[7]};
                    } else {
                        *reinterpret_cast<half8 *>(blk + kSegR + row * kD + col) =
                            half8{(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3],
                                  (_Float16)y[4], (_Float16)y[5], (_Float16)y[6], (_Float16)y[7]};
                    }
                }
            };
            lds_barrier();
#pragma unroll
            for (int e = 0; e < 16; ++e) hwc[e] = sCW[c4 * 16 + e];
            conv_v(0);
            lds_barrier();
            for (int c = 0; c <= last; ++c) {
                if (c + 1 < nch) conv_v(c + 1);  // nothing for a lane without a conv item
                const int oc = c - 3 - kSegLag;
                if (vtid >= 64 && vtid < 64 + kOutLanes && oc >= 0 && oc < nch) emit(oc);
                lds_barrier();
            }
            // raw v inputs of the sequence's last three tokens -> conv state out
            if (vh == 0 && a.conv && a.conv_state_out && lane < 3 * NCG && !mcol && seg == a.nseg - 1) {
                const int sidx = lane / NCG, cg = lane % NCG;
                const int tau = si.T - 3 + sidx;
                const int ch = 2 * a.Hk * kD + h * kD + sv0 + cg * 8;
                uint4 rw = make_uint4(0, 0, 0, 0);
                if (tau >= 0)
                    rw = *reinterpret_cast<const uint4 *>(a.v + ((si.tok0 + tau) * a.Hv + h) * kD + sv0 + cg * 8);
                else if (a.conv_state_in)
                    rw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + (3 + tau)) * a.Cc + ch);
                *reinterpret_cast<uint4 *>(a.conv_state_out + ((size_t)b * 3 + sidx) * a.Cc + ch) = rw;
            }
        }
        lds_barrier();
        // with no more items than workgroups, every item has a workgroup of its own (each one
        // that has not started yet takes one when it does), so a finished workgroup leaves
        if (a.n_items <= a.grid) break;
    }
    // the last workgroup out rewinds the queues for the next launch (its own ticket requests
    // have returned before its exit is counted, so relaxed order suffices here too)
    if (tid == 0) {
        const unsigned int done =
            __hip_atomic_fetch_add(a.exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == (unsigned int)a.grid - 1) {
            for (int q = 0; q < 8; ++q) __hip_atomic_store(a.tickets + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.exits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- two-level scan: the later passes

struct SegArgs {
    const float *state_in;   // [B Hv][128][128] or nullptr
    const float *seg_state;  // [B Hv nseg][128][256]: [M | N] of every segment
    _Float16 *seg_frag;      // [B Hv nseg][8 column tiles][4 k-steps][64 lanes][8]: start states as MFMA B operands
    float *state_out;        // [B Hv][128][128]
    const _Float16 *seg_out; // per (chunk slot, value head): R fragments and O0 rows (kSegBlk halves)
    const uint16_t *z, *norm_w;
    uint16_t *o;
    int B, T, Hv, nch, nseg, seg_chunks, norm;
    int out_cpw;             // chunks per workgroup of the output kernel (consecutive, one segment)
    float eps_norm;
};

// Start states of the segments and the final state, in fp32: S_0 = state_in,
// S_{p+1} = M_p S_p + N_p (each segment's map is affine in its start state).  One
// workgroup per (head, 16-column slice): the columns of a state never mix.  The start
// state of every segment is also written as MFMA operand fragments for the output pass.
// The products run on the fp32 MFMA (16x16x4): wave w owns rows 16 w .. 16 w + 15, and its
// lane l (row i = l % 16, quarter q = l / 16) brings the k-steps s = 0..31 of the contraction
// index k = 32 q + s, so that its A values are one contiguous piece of row 16 w + i of M.
// Two register sets hold those pieces (and the lane's N values) of segments p and p + 1; each
// is reloaded with segment p + 2 right after its last use, so the chain of segments waits on
// memory once.  Two accumulators split the 32 k-steps into independent MFMA chains.
// grid (B Hv 8), 512 threads
__global__ __launch_bounds__(512) void seg_combine_kernel(SegArgs a) {
    __shared__ float sS[kD][16 + 1];
    const int chain = blockIdx.x / kTiles, ct = blockIdx.x % kTiles;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, i = lane & 15, q = lane >> 4;
    auto mrow = [&](int p, int row) { return a.seg_state + (((size_t)chain * a.nseg + p) * kD + row) * (2 * kD); };
    // M[16 w + i][32 q .. 32 q + 31] and N[16 w + 4 q + v][16 ct + i] of segment p (clamped)
    auto fetch = [&](int p, float4 (&m)[8], float (&n)[4]) __attribute__((always_inline)) {
        const int pc = min(p, a.nseg - 1);
        const float *M = mrow(pc, 16 * w + i) + 32 * q;
#pragma unroll
        for (int u = 0; u < 8; ++u) m[u] = *reinterpret_cast<const float4 *>(M + 4 * u);
#pragma unroll
        for (int v = 0; v < 4; ++v) n[v] = mrow(pc, 16 * w + 4 * q + v)[kD + 16 * ct + i];
    };
    // the start state first (the first step waits for it alone), then both register sets
    float s0[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int x = tid + 512 * e, rr = x / 16, j = x % 16;
        s0[e] = a.state_in ? a.state_in[((size_t)chain * kD + rr) * kD + 16 * ct + j] : 0.0f;
    }
    float4 mA[8], mB[8];
    float nA[4], nB[4];
    fetch(0, mA, nA);
    fetch(1, mB, nB);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int x = tid + 512 * e;
        sS[x / 16][x % 16] = s0[e];
    }
    __syncthreads();
    auto step = [&](int p, float4 (&m)[8], float (&n)[4]) __attribute__((always_inline)) {
        const size_t vc = (size_t)chain * a.nseg + p;
        if (tid < 256) {  // fragment ks of column tile ct: lane L holds column l16 at rows 32 ks + {4 lq + e, 16 + 4 lq + e}
            const int ks = tid >> 6, L = tid & 63, l16 = L & 15, lq = L >> 4;
            half8 f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = (_Float16)sS[32 * ks + 4 * lq + e][l16];
                f[4 + e] = (_Float16)sS[32 * ks + 16 + 4 * lq + e][l16];
            }
            *reinterpret_cast<half8 *>(a.seg_frag + (((vc * kTiles + ct) * 4 + ks) * 64 + L) * 8) = f;
        }
        // D rows 16 w + 4 q + v, column i: N plus the two chains
        floatx4 acc0 = {n[0], n[1], n[2], n[3]}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; u += 2) {
            const int k = 32 * q + 4 * u;
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[u].x, sS[k][i], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[u + 1].x, sS[k + 4][i], acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[u].y, sS[k + 1][i], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[u + 1].y, sS[k + 5][i], acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[u].z, sS[k + 2][i], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[u + 1].z, sS[k + 6][i], acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[u].w, sS[k + 3][i], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[u + 1].w, sS[k + 7][i], acc1, 0, 0, 0);
        }
        fetch(p + 2, m, n);  // this set's next segment, past the last use
        __syncthreads();
#pragma unroll
        for (int v = 0; v < 4; ++v) sS[16 * w + 4 * q + v][i] = acc0[v] + acc1[v];
        __syncthreads();
    };
    for (int p = 0; p < a.nseg; p += 2) {
        step(p, mA, nA);
        if (p + 1 < a.nseg) step(p + 1, mB, nB);
    }
    for (int x = tid; x < kD * 16; x += 512) {
        const int rr = x / 16, jj = x % 16;
        a.state_out[((size_t)chain * kD + rr) * kD + 16 * ct + jj] = sS[rr][jj];
    }
}

// Outputs of the two-level scan: O = O0 + R S_p for chunk c of segment p (R [64][128]
// times the start state, on MFMA), then the gated RMSNorm and the bf16 store.  A workgroup
// takes out_cpw consecutive chunks of one segment and head and keeps the segment's start
// state (32 B-operand fragments, 32 KB) in LDS across them; the next chunk's R, O0 and z are
// in flight while one is computed.  Wave w owns rows 16 w .. 16 w + 15 of a
// chunk; a row's 128 columns sit in 16 lanes.  O0, z and the outputs pass through LDS so
// that every global access is a 16-byte row piece.
// grid (B Hv nseg pieces), 256 threads
__global__ __launch_bounds__(256) void seg_output_kernel(SegArgs a) {
    __shared__ _Float16 sX[kC][kD + 8];  // O0, then the bf16 outputs
    __shared__ uint16_t sZ[kC][kD + 8];  // z
    __shared__ half8 sF[32][64];         // start-state fragment (column tile ct, k-step ks) at 4 ct + ks
    const int npiece = (a.seg_chunks + a.out_cpw - 1) / a.out_cpw;
    int id = blockIdx.x;
    const int piece = id % npiece;
    id /= npiece;
    const int p = id % a.nseg;
    id /= a.nseg;
    const int h = id % a.Hv, b = id / a.Hv;
    const int c_begin = p * a.seg_chunks + piece * a.out_cpw;
    const int c_end = min(min(c_begin + a.out_cpw, (p + 1) * a.seg_chunks), a.nch);
    if (c_begin >= c_end) return;  // the last segment is shorter (uniform over the workgroup)
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
    const size_t vc = ((size_t)b * a.Hv + h) * a.nseg + p;
    {
        const half8 *fr = reinterpret_cast<const half8 *>(a.seg_frag) + vc * kTiles * 4 * 64;
#pragma unroll
        for (int u = 0; u < 8; ++u) sF[8 * w + u][lane] = fr[(8 * w + u) * 64 + lane];
    }
    // the chunk's O0 rows and z rows of this thread (4 pieces each) and its wave's R fragments:
    // once chunk c's are in LDS (and R in named registers), the set is reloaded with chunk c + 1
    // (past the last chunk, the last one's again), in flight while chunk c is computed
    uint4 oP[4], zP[4], aP[4];
    auto load_chunk = [&](int c, uint4 (&xo)[4], uint4 (&xz)[4], uint4 (&xa)[4]) __attribute__((always_inline)) {
        const size_t gc = (size_t)b * a.nch + c, row0 = (size_t)b * a.T + (size_t)c * kC;
        const int nrows = min(kC, a.T - c * kC);
        const _Float16 *blk = a.seg_out + (gc * a.Hv + h) * kSegBlk;
        // z rows through a buffer resource over the chunk's rows: rows past T (and every row
        // without the norm, where z is absent) read as zero, with no branch around the loads
        const __amdgpu_buffer_rsrc_t rz =
            make_rsrc(a.norm ? a.z + (row0 * a.Hv + h) * kD : a.o, a.norm ? (unsigned int)nrows * a.Hv * kD * 2 : 0u);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(blk, kSegBlk * 2);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = tid + 256 * u, row = i >> 4, c8 = (i & 15) * 8;
            xo[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, (kSegR + row * kD + c8) * 2, 0, 0));
            xz[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rz, (row * a.Hv * kD + c8) * 2, 0, 0));
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            xa[ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, ((w * 4 + ks) * 64 + lane) * 16, 0, 0));
    };
    auto do_chunk = [&](int c, uint4 (&xo)[4], uint4 (&xz)[4], uint4 (&xa)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = tid + 256 * u, row = i >> 4, c8 = (i & 15) * 8;
            *reinterpret_cast<uint4 *>(&sX[row][c8]) = xo[u];
            *reinterpret_cast<uint4 *>(&sZ[row][c8]) = xz[u];
        }
        const half8 A0 = __builtin_bit_cast(half8, xa[0]), A1 = __builtin_bit_cast(half8, xa[1]),
                    A2 = __builtin_bit_cast(half8, xa[2]), A3 = __builtin_bit_cast(half8, xa[3]);
        load_chunk(min(c + 1, c_end - 1), xo, xz, xa);
        __syncthreads();
        floatx4 acc[8];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            acc[ct] = mfma16x16x32(A0, sF[4 * ct][lane], floatx4{0.f, 0.f, 0.f, 0.f});
            acc[ct] = mfma16x16x32(A1, sF[4 * ct + 1][lane], acc[ct]);
            acc[ct] = mfma16x16x32(A2, sF[4 * ct + 2][lane], acc[ct]);
            acc[ct] = mfma16x16x32(A3, sF[4 * ct + 3][lane], acc[ct]);
        }
        float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * w + 4 * lq + e;
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                acc[ct][e] += (float)sX[row][16 * ct + l16];
                ss[e] += acc[ct][e] * acc[ct][e];
            }
        }
        __syncthreads();  // sX is reused for the outputs
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * w + 4 * lq + e;
            const float rstd = __builtin_amdgcn_rsqf(row16_sum(ss[e]) * (1.0f / kD) + a.eps_norm);
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const int col = 16 * ct + l16;
                float y = acc[ct][e];
                if (a.norm) y = bf16_to_f32(a.norm_w[col]) * (y * rstd) * silu(bf16_to_f32(sZ[row][col]));
                reinterpret_cast<uint16_t *>(&sX[row][0])[col] = f32_to_bf16(y);
            }
        }
        __syncthreads();
        const size_t row0 = (size_t)b * a.T + (size_t)c * kC;
        const int nrows = min(kC, a.T - c * kC);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = tid + 256 * u, row = i >> 4, c8 = (i & 15) * 8;
            if (row < nrows)
                *reinterpret_cast<uint4 *>(a.o + ((row0 + row) * a.Hv + h) * kD + c8) =
                    *reinterpret_cast<const uint4 *>(&sX[row][c8]);
        }
        __syncthreads();  // the next chunk's O0 and z overwrite sX and sZ
    };
    load_chunk(c_begin, oP, zP, aP);
    for (int c = c_begin; c < c_end; ++c) do_chunk(c, oP, zP, aP);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct ChainLaunch {
    const void *fn;
    size_t lds;
    int grid, ncu;
};

// Two-level scan planning: the chip's compute units (MI355X) and the shortest segment.
constexpr int kSegChipCUs = 256;
constexpr int kSegMinChunks = 16;
// Where the sequential pass would fill up to half of the chip (16-column slices of 9 to 16
// chains), two segments fill all of it.  The segment pass runs half the chunks at a similar
// pace per chunk, and the combine and output kernels add about 30 us, so the split pays from
// about 64 chunks on.  0.8B-shaped layer (64 chunks, 16 chains): sequential pass 118 us against
// segment pass 54 us + combine 11 us + outputs 21 us.
constexpr int kSegMinChunksHalf = 32;

// What a launch needs to know about a device and a kernel, found on first use and kept
// (the queries cost tens of microseconds of host time per call otherwise).
struct DeviceFacts {
    std::mutex mu;
    int ncu = 0;
    int seg_per_cu = 0;  // resident workgroups per CU of the two-level scan's first pass
    int prep_lds = 0;    // dynamic LDS limit set so far for the prep kernel
};

int device_facts(DeviceFacts **out) {
    static DeviceFacts per_dev[64];
    int dev = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return fail("hipGetDevice", e);
    if (dev < 0 || dev >= 64) return fail("prefill: device index out of range");
    *out = &per_dev[dev];
    return 0;
}

// Launch shape of the two-level scan's first pass: as many workgroups as items, at most
// one round of resident ones (no workgroup waits for another, so any number runs correctly).
int seg_launch_shape(const SegPassArgs &a, ChainLaunch *cl) {
    constexpr size_t lds = ChainLds<kSegNT>::bytes;
    const void *fn = reinterpret_cast<const void *>(segment_pass_kernel);
    DeviceFacts *df;
    int rc = device_facts(&df);
    if (rc) return rc;
    int ncu, per_cu;
    {
        std::lock_guard<std::mutex> g(df->mu);
        hipError_t e;
        if (!df->ncu) {
            int dev = 0;
            if ((e = hipGetDevice(&dev)) != hipSuccess) return fail("hipGetDevice", e);
            if ((e = hipDeviceGetAttribute(&df->ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
                return fail("hipDeviceGetAttribute(multiprocessor count)", e);
        }
        if (!df->seg_per_cu) {
            if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
                return fail("hipFuncSetAttribute(segment_pass_kernel)", e);
            if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&df->seg_per_cu, fn, 512, lds)) != hipSuccess)
                return fail("hipOccupancyMaxActiveBlocksPerMultiprocessor(segment_pass_kernel)", e);
        }
        ncu = df->ncu;
        per_cu = df->seg_per_cu;
    }
    const int cap = ncu * per_cu;
    if (cap < 1) return fail("segment_pass_kernel: no resident workgroup fits a compute unit");
    cl->fn = fn;
    cl->lds = lds;
    cl->grid = a.n_items < cap ? a.n_items : cap;
    cl->ncu = ncu;
    return 0;
}

} // namespace

int plan_prefill(int B, int T, int Hk, int Hv, bool packed, int segments, PrefillPlan *plan) {
    const long long chains = (long long)B * Hv;
    // 16-column slices while the heads leave most of the chip idle, 32-column slices beyond
    const int nsl = chains <= 32 ? 8 : 4;
    plan->nslice = nsl;
    plan->nt = kTiles / nsl;
    plan->bv = 16 * plan->nt;
    plan->nchunks = (T + kC - 1) / kC;
    // packed: sequence b's chunks from slot floor(cu[b] / 64) + b on, all below floor(T / 64) + B
    plan->nslots = packed ? (long long)(T / kC) + B : (long long)B * plan->nchunks;
    // one row of mailbox words per (sequence, value head, slice, ring slot), and one more set
    // past them that the sequential pass publishes into outside a sequence's chunk range
    plan->mbox_bytes = align256((size_t)(chains + 1) * kTiles * kMboxRing * kC * sizeof(unsigned long long));
    plan->xch_bytes = kHeaderBytes + plan->mbox_bytes;
    plan->qk_bytes = align256((size_t)plan->nslots * Hk * kQKF * sizeof(_Float16));
    plan->tp_bytes = align256((size_t)plan->nslots * Hv * kTPF * sizeof(_Float16));
    // Two-level scan (even batches): worth it when the sequential pass would leave much of the
    // chip idle (few heads) and the sequences are long.  Its first pass runs 256 columns per
    // head in slices of 32 (measured on the shapes it is for: as many 32-column slices as fit
    // the chip beat half as many segments in 16-column slices, at about 2 us against 1.25 us per
    // chunk), so nseg segments keep B Hv 8 nseg workgroups busy; nseg fills one round of the
    // chip (two segments where the sequential pass would fill half of it).  `segments`
    // overrides the choice (1: never, n >= 2: n segments).
    plan->nseg = 1;
    plan->seg_chunks = plan->nchunks;
    if (!packed) {
        long long want = 0;
        if (segments > 0)
            want = segments;
        else if (chains * nsl * 4 <= kSegChipCUs)  // the sequential pass would use at most a quarter of the chip
            want = std::min<long long>(kSegChipCUs / (chains * 8), plan->nchunks / kSegMinChunks);
        else if (chains * 8 * 2 <= kSegChipCUs)  // at most half of it: two segments, if they are long
            want = std::min<long long>(2, plan->nchunks / kSegMinChunksHalf);
        want = std::min<long long>(want, plan->nchunks);
        if (want >= 2) {
            plan->seg_chunks = (int)((plan->nchunks + want - 1) / want);
            plan->nseg = (plan->nchunks + plan->seg_chunks - 1) / plan->seg_chunks;
            plan->nslice = 4;  // 32-column slices in the segment pass
            plan->nt = 2;
            plan->bv = 32;
        }
    }
    plan->seg_out_bytes = plan->seg_state_bytes = plan->seg_frag_bytes = 0;
    if (plan->nseg > 1) {
        const size_t vchains = (size_t)chains * plan->nseg;
        plan->seg_out_bytes = align256((size_t)B * plan->nchunks * Hv * kSegBlk * sizeof(_Float16));
        plan->seg_state_bytes = align256(vchains * kD * 2 * kD * sizeof(float));
        plan->seg_frag_bytes = align256(vchains * kTiles * 4 * kFrag * sizeof(_Float16));
    }
    plan->total_bytes = plan->xch_bytes + plan->qk_bytes + plan->tp_bytes + plan->seg_out_bytes +
                        plan->seg_state_bytes + plan->seg_frag_bytes;
    return 0;
}

PrefillRegions prefill_regions(void *workspace, const PrefillPlan &plan, int B, int Hv) {
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    PrefillRegions r;
    r.err = reinterpret_cast<unsigned int *>(ws + kErrOffset);
    r.tickets = reinterpret_cast<unsigned int *>(ws + kTicketOffset);
    r.exits = reinterpret_cast<unsigned int *>(ws + kExitOffset);
    r.mbox = reinterpret_cast<unsigned long long *>(ws + kHeaderBytes);
    r.qkf = reinterpret_cast<_Float16 *>(ws + plan.xch_bytes);
    r.tpf = reinterpret_cast<_Float16 *>(ws + plan.xch_bytes + plan.qk_bytes);
    r.seg = ws + plan.xch_bytes + plan.qk_bytes + plan.tp_bytes;
    (void)B;
    (void)Hv;
    return r;
}

// Two kernels one after the other on the caller's stream: the prep kernel (every chunk of
// every key head in parallel; it also clears the workspace's exchange area), then the
// sequential pass, whose workgroups only ever wait for sibling workgroups of the same
// launch.  With the two-level scan the sequential pass is its first pass, followed by the
// combine and output kernels.
int launch_prefill(const PrefillParams &p, const PrefillPlan &plan, hipStream_t stream) {
    const PrefillRegions rg = prefill_regions(p.workspace, plan, p.B, p.Hv);
    const size_t chains = (size_t)p.B * p.Hv;
    hipError_t e;
    int rc;

    PrepArgs pa;
    pa.q = p.q; pa.k = p.k; pa.conv_w = p.conv_w; pa.conv_state_in = p.conv_state_in;
    pa.g = p.g; pa.beta = p.beta; pa.A_log = p.A_log; pa.dt_bias = p.dt_bias; pa.conv_state_out = p.conv_state_out;
    pa.qkf = rg.qkf; pa.tpf = rg.tpf; pa.cu = p.cu_seqlens;
    pa.clear = reinterpret_cast<uint4 *>(p.workspace); pa.clear_n16 = plan.xch_bytes / 16;
    pa.B = p.B; pa.T = p.T; pa.Hk = p.Hk; pa.Hv = p.Hv; pa.r = p.Hv / p.Hk;
    pa.Cc = 2 * p.Hk * kD + p.Hv * kD; pa.conv = p.conv_width == 4; pa.nch = plan.nchunks;
    pa.eps_l2 = p.eps_l2;
    const size_t plds = PrepLds::bytes(pa.r);
    const void *prep_fn = reinterpret_cast<const void *>(chunk_prep_kernel);
    {   // raise the prep kernel's LDS limit when this head ratio needs more than set so far
        DeviceFacts *df;
        if ((rc = device_facts(&df))) return rc;
        std::lock_guard<std::mutex> g(df->mu);
        if ((int)plds > df->prep_lds) {
            if ((e = hipFuncSetAttribute(prep_fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)plds)) != hipSuccess)
                return fail("hipFuncSetAttribute(chunk_prep_kernel)", e);
            df->prep_lds = (int)plds;
        }
    }
    void *pargs[] = {&pa};
    if ((e = hipLaunchKernel(prep_fn, dim3((unsigned)(plan.nslots * p.Hk)), dim3(256), pargs, plds, stream)) !=
        hipSuccess)
        return fail("hipLaunchKernel(chunk_prep_kernel)", e);

    if (plan.nseg <= 1) return launch_pass(p, plan, rg, stream);

    // ---- two-level scan
    SegPassArgs a;
    a.qkf = rg.qkf; a.tpf = rg.tpf;
    a.v = p.v; a.conv_w = p.conv_w; a.conv_state_in = p.conv_state_in; a.conv_state_out = p.conv_state_out;
    a.tickets = rg.tickets; a.exits = rg.exits;
    a.B = p.B; a.T = p.T; a.Hk = p.Hk; a.Hv = p.Hv; a.r = pa.r; a.Cc = pa.Cc; a.conv = pa.conv;
    a.nch = plan.nchunks; a.grid = 0;
    a.seg_out = reinterpret_cast<_Float16 *>(rg.seg);
    a.seg_state = reinterpret_cast<float *>(rg.seg + plan.seg_out_bytes);
    a.nseg = plan.nseg; a.seg_chunks = plan.seg_chunks;
    a.n_items = (int)(chains * plan.nseg * 2 * plan.nslice);
    ChainLaunch cl;
    if ((rc = seg_launch_shape(a, &cl))) return rc;
    a.grid = cl.grid;
    void *cargs[] = {&a};
    if ((e = hipLaunchKernel(cl.fn, dim3(cl.grid), dim3(512), cargs, cl.lds, stream)) != hipSuccess)
        return fail("hipLaunchKernel(segment_pass_kernel)", e);
    SegArgs sa;
    sa.state_in = p.state_in; sa.seg_state = a.seg_state;
    sa.seg_frag = reinterpret_cast<_Float16 *>(rg.seg + plan.seg_out_bytes + plan.seg_state_bytes);
    sa.state_out = p.state_out; sa.seg_out = a.seg_out; sa.z = p.z; sa.norm_w = p.norm_w; sa.o = p.o;
    sa.B = p.B; sa.T = p.T; sa.Hv = p.Hv; sa.nch = plan.nchunks; sa.nseg = plan.nseg;
    sa.seg_chunks = plan.seg_chunks; sa.norm = p.norm; sa.eps_norm = p.eps_norm;
    // output workgroups: up to 8 chunks each, while at least two per CU of the chip remain
    const long long chunk_heads = (long long)chains * plan.nseg * plan.seg_chunks;
    sa.out_cpw = (int)std::max<long long>(1, std::min<long long>(8, chunk_heads / (2 * kSegChipCUs)));
    const long long out_grid = (long long)chains * plan.nseg * ((plan.seg_chunks + sa.out_cpw - 1) / sa.out_cpw);
    void *sargs[] = {&sa};
    if ((e = hipLaunchKernel(reinterpret_cast<const void *>(seg_combine_kernel), dim3((unsigned)(chains * kTiles)),
                             dim3(512), sargs, 0, stream)) != hipSuccess)
        return fail("hipLaunchKernel(seg_combine_kernel)", e);
    if ((e = hipLaunchKernel(reinterpret_cast<const void *>(seg_output_kernel), dim3((unsigned)out_grid), dim3(256),
                             sargs, 0, stream)) !=
        hipSuccess)
        return fail("hipLaunchKernel(seg_output_kernel)", e);
    return 0;
}

} // namespace gdn
