// gdn_pass.hip -- the sequential pass of the chunked prefill on gfx950 (steps a6-a8):
// the state chain over the chunks of each (sequence, value head), the read-out of every
// chunk and the gated RMSNorm, fed by the chunk operands that chunk_prep_kernel wrote to
// the workspace before this kernel starts.
//
// Math ("How Qwen3.5 works" §9.11).  Per chunk of 64 tokens with start state S (K-major
// 128 x 128 fp32), cumulative log-decay G and the prep kernel's T diag(beta) and
// P = (Q K^T) o R:
//   X     = V - diag(e^G) K S
//   Delta = T diag(beta) X
//   O     = diag(e^G) Q S + P Delta
//   S'    = e^{G_C} S + K^T diag(e^{G_C - G}) Delta
// then y = w * O / rms(O) * silu(z) per output row (model spec node gdn.norm).
//
// One workgroup of 8 waves per (sequence, value head, slice of 16 NT value columns); the
// columns of a state evolve independently, so a head runs as 8 / NT slices on as many
// compute units.  Measured on gfx950, one wave streams about 27 B/clk from LDS with
// 16-byte reads, 16 B/clk with the transposing read and about 21 B/clk from L2, and a
// compute unit takes about 64 B/clk from L2, while one 16x16x32 MFMA every 16 clocks
// consumes a 1 KB A operand.  So every operand stream has exactly one consumer and one
// path, and each fragment a wave loads feeds NT MFMAs:
//   wave 0  state: the slice's state in accumulators; k^ fragments from LDS, k^T
//           fragments straight from the workspace into registers a chunk ahead (the prep
//           kernel stores both orientations), T diag(beta) and the decays from LDS.
//   wave 1  read-out: q^ fragments, P and e^G straight from the workspace a chunk ahead;
//           S and Delta of the chunk from the state wave through LDS.
//   waves 2..7 helpers: helper 0 the per-row sums of squares the gated norm needs from
//           every slice of a head (tagged words in a workspace mailbox, bounded waits);
//           helper 1 the DMA of the k^ fragments, T diag(beta) / decays and raw v rows into
//           LDS rings; helpers 2..5 conv + SiLU of v and the gated RMSNorm with the bf16 store.
// One LDS barrier per iteration hands data between the roles; every hand-off is at least
// one barrier away.  Work items (head, slice) come from eight ticket queues, one per XCD,
// grouped by key head so that the slices reading one key head's operands share an L2.
#include <algorithm>
#include <mutex>

#include "gdn_internal.h"
#include "gdn_prefill_common.h"

namespace gdn {
namespace {

constexpr int kLagP = 2;            // iterations between publishing a chunk's row sums and reading the siblings'
constexpr int kORingP = kLagP + 3;  // pre-norm output tiles held in LDS
static_assert(kMboxRing > 2 * kLagP + 1, "a mailbox slot must outlive the slowest sibling's read");
constexpr int kTB = 7 * 1024;       // bytes of T diag(beta) fragments and decay vectors (head of a tpf block)
constexpr int kSDT = 6 * 1024;      // bytes per tile of Sb (4 fragments) and Delta (2 fragments)

// (m & a) | (~m & b) on the bit patterns: a when m is all-ones, b when it is zero
__device__ __forceinline__ float bit_select(unsigned int m, float a, float b) {
    return __uint_as_float((m & __float_as_uint(a)) | (~m & __float_as_uint(b)));
}

struct PassArgs {
    const _Float16 *qkf, *tpf;
    const uint16_t *v, *z, *conv_w, *norm_w, *conv_state_in;
    const float *state_in;
    uint16_t *o, *conv_state_out;
    float *state_out;
    unsigned long long *mbox;  // [B Hv][8 slices][kMboxRing][64]: tagged per-row partial sums of squares
    unsigned int *err;         // error word (bit 0: a bounded wait timed out; bit 1: a packed sequence skipped)
    unsigned int *tickets;     // [8] next item of each XCD queue
    const int *cu;             // packed sequences: [B + 1] token offsets (nullptr: even batch)
    int B, T, Hk, Hv, r, Cc, conv, norm, nch;
    float eps_norm;
};

template <int NT>
struct PassLds {
    static constexpr int BV = 16 * NT;              // value columns of the slice
    static constexpr int VT = BV * PL;              // floats of one column-major [BV][PL] output tile
    static constexpr int NRD = kC * BV * 2 / 1024;  // DMA instructions for 64 raw v rows of the slice
    static constexpr int SVT = vtile(BV);           // fp16 of one conv(v) buffer
    static constexpr size_t sK = 0;                                // [3][16 KB] k^ fragments
    static constexpr size_t sTB = sK + 3 * 16 * 1024;              // [3][kTB]   T diag(beta) fragments, decays
    static constexpr size_t sSD = sTB + 3 * kTB;                   // [2][NT][kSDT] Sb, Delta per tile
    static constexpr size_t sV = sSD + 2 * NT * kSDT;              // fp16 [2][SVT] conv(v), columns at vcol
    static constexpr size_t sO = sV + 2 * 2 * SVT;                 // fp32 [kORingP][BV][PL] pre-norm output, rows at orow
    static constexpr size_t sRawV = sO + 4 * kORingP * VT;         // bf16 [3][64][BV] raw v
    static constexpr size_t sHalo = sRawV + 2 * 3 * kC * BV;       // bf16 [2][3][BV] raw v rows before a chunk
    static constexpr size_t sRstd = sHalo + 2 * 2 * 3 * BV;        // fp32 [2][64] 1/rms
    static constexpr size_t sCW = sRstd + 4 * 2 * kC;              // fp32 [BV][4] conv taps of the v channels
    static constexpr size_t sNW = sCW + 4 * 4 * BV;                // fp32 [BV] gated-norm weights
    static constexpr size_t bytes = sNW + 4 * BV;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    static_assert(sO % 16 == 0 && sRawV % 16 == 0 && sHalo % 16 == 0, "16-byte LDS alignment");
};

// One chunk of the state chain for the NT tiles of the slice.
//   S    [t][ti]: tile t, key-row tile ti, accumulator layout (col l16, rows 16 ti + 4 lq + e)
//   fkT  k^T fragments of this chunk (row tile ti = f >> 1, token k-step f & 1); each is
//        reloaded from rnext (the next chunk's block, or this one's past the last chunk)
//        right after its last use.  The reloads are unconditional: with a branch around
//        them the compiler's count of outstanding loads turns conservative and it waits for
//        loads issued in the same pass, which exposes their whole latency.
template <int NT>
__device__ __forceinline__ void state_chunk(const unsigned char *smem, floatx4 (&S)[NT][8], half8 (&fkT)[16],
                                            __amdgpu_buffer_rsrc_t rnext, int c, int lane, int l16, int lq) {
    using L = PassLds<NT>;
    const unsigned char *kb = smem + L::sK + (c % 3) * 16384 + lane * 16;
    const unsigned char *tb = smem + L::sTB + (c % 3) * kTB;
    const _Float16 *sVc = reinterpret_cast<const _Float16 *>(smem + L::sV) + (c & 1) * L::SVT;
    half8 *sd = reinterpret_cast<half8 *>(const_cast<unsigned char *>(smem) + L::sSD + (c & 1) * NT * kSDT) + lane;

    // With one tile there are registers to spare: T diag(beta) of the chunk is then requested
    // first, so that its LDS latency hides behind the K S products (with two tiles the extra
    // 24 registers would spill)
    const float4 *dec = reinterpret_cast<const float4 *>(tb + 6 * 1024);  // e^G [64], e^{G_C - G} [64], e^{G_C}
    half8 tbf[6];
    if constexpr (NT == 1) {
#pragma unroll
        for (int f = 0; f < 6; ++f) tbf[f] = *reinterpret_cast<const half8 *>(tb + f * 1024 + lane * 16);
    }
    // K S over the four 32-key steps.  Each step's fp16 S fragments go to LDS for the read-out
    // wave as soon as they are packed, so they are packed once.  LDS operations complete in
    // order, so the next step's k^ reads queue behind these stores; measured, that costs less
    // than packing S a second time after the chunk's last read (27B-shaped pass, median
    // 6.49 against 6.55 ms).  Delta goes to LDS after the chunk's last read.
    floatx4 ks[4][NT];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int t = 0; t < NT; ++t) ks[I][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        half8 a[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) a[I] = *reinterpret_cast<const half8 *>(kb + (4 * I + s2) * 1024);
        half8 sb[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            sb[t] = pack_tiles(S[t][2 * s2], S[t][2 * s2 + 1]);
            sd[t * (kSDT / 16) + 64 * s2] = sb[t];  // the fp16 S before the chunk, for the read-out
        }
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int t = 0; t < NT; ++t) ks[I][t] = mfma16x16x32(a[I], sb[t], ks[I][t]);
    }
    // X = V - e^G K S
    half8 Xb[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        floatx4 X[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const float4 eg = dec[4 * I + lq];
            const half4 vv = lds_half4(sVc + vcol(16 * t + l16) + 16 * I + 4 * lq);
            X[I][0] = (float)vv[0] - eg.x * ks[I][t][0];
            X[I][1] = (float)vv[1] - eg.y * ks[I][t][1];
            X[I][2] = (float)vv[2] - eg.z * ks[I][t][2];
            X[I][3] = (float)vv[3] - eg.w * ks[I][t][3];
        }
        Xb[t][0] = pack_tiles(X[0], X[1]);
        Xb[t][1] = pack_tiles(X[2], X[3]);
    }
    // Delta = T diag(beta) X (lower triangular: rows 0..31 use the first 32 tokens only)
    if constexpr (NT != 1) {
#pragma unroll
        for (int f = 0; f < 6; ++f) tbf[f] = *reinterpret_cast<const half8 *>(tb + f * 1024 + lane * 16);
    }
    // e^{G_C - G} and e^{G_C}: the chunk's last LDS reads
    float4 egc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) egc[u] = dec[16 + 4 * u + lq];
    const float dC = reinterpret_cast<const float *>(tb + 6 * 1024)[2 * kC];
    half8 Dsb[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        floatx4 d[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) d[I] = floatx4{0.f, 0.f, 0.f, 0.f};
        d[0] = mfma16x16x32(tbf[0], Xb[t][0], d[0]);
        d[1] = mfma16x16x32(tbf[1], Xb[t][0], d[1]);
        d[2] = mfma16x16x32(tbf[2], Xb[t][0], d[2]);
        d[2] = mfma16x16x32(tbf[3], Xb[t][1], d[2]);
        d[3] = mfma16x16x32(tbf[4], Xb[t][0], d[3]);
        d[3] = mfma16x16x32(tbf[5], Xb[t][1], d[3]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            sd[t * (kSDT / 16) + 64 * (4 + s)] = pack_tiles(d[2 * s], d[2 * s + 1]);
            const float4 c0 = egc[2 * s], c1 = egc[2 * s + 1];
            Dsb[t][s] = half8{(_Float16)(d[2 * s][0] * c0.x), (_Float16)(d[2 * s][1] * c0.y),
                              (_Float16)(d[2 * s][2] * c0.z), (_Float16)(d[2 * s][3] * c0.w),
                              (_Float16)(d[2 * s + 1][0] * c1.x), (_Float16)(d[2 * s + 1][1] * c1.y),
                              (_Float16)(d[2 * s + 1][2] * c1.z), (_Float16)(d[2 * s + 1][3] * c1.w)};
        }
    }
    // S = e^{G_C} S + K^T Delta~, each k^T fragment used for every tile, then reloaded.  The
    // token step is the outer loop, so 8 NT independent accumulations separate the two
    // products into one accumulator.
#pragma unroll
    for (int ti = 0; ti < 8; ++ti)
#pragma unroll
        for (int t = 0; t < NT; ++t) S[t][ti] = S[t][ti] * dC;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int ti = 0; ti < 8; ++ti) {
#pragma unroll
            for (int t = 0; t < NT; ++t) S[t][ti] = mfma16x16x32(fkT[2 * ti + s], Dsb[t][s], S[t][ti]);
            fkT[2 * ti + s] = ld_frag(rnext, lane * 16, 2 * ti + s);
        }
    }
}

// Read-out of one chunk for the NT tiles: O = e^G (Q S) + P Delta, to LDS (column-major).
// fq holds the q^ fragments, fp the P fragments and eg the e^G rows of this chunk; each is
// reloaded (unconditionally, as in state_chunk) from rq / rt right after its last use.
template <int NT>
__device__ __forceinline__ void readout_chunk(unsigned char *smem, half8 (&fq)[16], half8 (&fp)[6], float4 (&eg)[4],
                                              __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rt, int c, int lane,
                                              int l16, int lq) {
    using L = PassLds<NT>;
    const half8 *sd = reinterpret_cast<const half8 *>(smem + L::sSD + (c & 1) * NT * kSDT) + lane;
    float *sOc = reinterpret_cast<float *>(smem + L::sO) + (c % kORingP) * L::VT;
    // Q S, k-step outermost: each S fragment is read from LDS once and serves the four row tiles
    floatx4 qs[4][NT];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int t = 0; t < NT; ++t) qs[I][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        half8 Sb[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) Sb[t] = sd[t * (kSDT / 16) + 64 * s2];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int t = 0; t < NT; ++t) qs[I][t] = mfma16x16x32(fq[4 * I + s2], Sb[t], qs[I][t]);
            fq[4 * I + s2] = ld_frag(rq, lane * 16, 4 * I + s2);
        }
    }
    half8 Db[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) Db[t][s] = sd[t * (kSDT / 16) + 64 * (4 + s)];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            floatx4 ot = {qs[I][t][0] * eg[I].x, qs[I][t][1] * eg[I].y, qs[I][t][2] * eg[I].z, qs[I][t][3] * eg[I].w};
            if (I < 2) {
                ot = mfma16x16x32(fp[I], Db[t][0], ot);
            } else {
                ot = mfma16x16x32(fp[2 + 2 * (I - 2)], Db[t][0], ot);
                ot = mfma16x16x32(fp[3 + 2 * (I - 2)], Db[t][1], ot);
            }
            const int j = 16 * t + l16;
            *reinterpret_cast<float4 *>(sOc + j * PL + orow(L::BV, 16 * I + 4 * lq, j)) = make_float4(ot[0], ot[1], ot[2], ot[3]);
        }
    }
#pragma unroll
    for (int f = 0; f < 6; ++f) fp[f] = ld_frag(rt, kPOff * 2 + lane * 16, f);
#pragma unroll
    for (int I = 0; I < 4; ++I) eg[I] = ld_f4(rt, kVecOff * 2 + lq * 16, 64 * I);
}

// grid: min(items, resident slots), 512 threads
template <int NT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void pass_kernel(PassArgs a) {
    using L = PassLds<NT>;
    constexpr int BV = L::BV, VT = L::VT, NRD = L::NRD;
    constexpr int NSL = kTiles / NT;  // slices per head
    constexpr int NCG = BV / 8;       // 8-column groups of a slice row
    // conv items: RPI consecutive rows of 4 channels per lane, on helpers 0..NCV-1
    constexpr int RPI = 2;
    constexpr int NC4 = BV / 4;
    constexpr int NCONV = (kC / RPI) * NC4;  // 128 (NT = 1) or 256 (NT = 2)
    constexpr int NCV = NCONV / 64;          // conv helpers
    // gating items: one row piece of 8 columns per lane and iteration, on helpers 6 - NGT .. 5
    constexpr int NGATE = kC * NCG;          // 128 or 256
    constexpr int NGT = 4;                   // gating helpers
    constexpr int GPL = (NGATE + 64 * NGT - 1) / (64 * NGT);  // items per gating lane (1 or 2)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Helper index (0..5) of waves 2..7.  A workgroup's waves go to the four SIMDs in turn, so
    // waves 4 and 5 share a SIMD with the state and the read-out wave: they take the two light
    // roles (DMA, exchange), and the four conv + gating helpers get SIMDs 2 and 3 to themselves.
    const int hidx = wave == 4 ? 1 : wave == 5 ? 0 : wave < 4 ? wave : wave - 2;
    float *sO = reinterpret_cast<float *>(smem + L::sO);
    uint16_t *sRawV = reinterpret_cast<uint16_t *>(smem + L::sRawV);
    uint16_t *sHalo = reinterpret_cast<uint16_t *>(smem + L::sHalo);
    _Float16 *sV = reinterpret_cast<_Float16 *>(smem + L::sV);
    float *sRstd = reinterpret_cast<float *>(smem + L::sRstd);
    float *sCW = reinterpret_cast<float *>(smem + L::sCW);
    float *sNW = reinterpret_cast<float *>(smem + L::sNW);
    __shared__ int s_item;

    const int xcc = static_cast<int>(xcc_id() & 7u);
    const int ngroups = a.B * a.Hk;  // (sequence, key head) groups; group g sits in queue g % 8
    const int per_group = a.r * NSL;
    int qi = 0;

    for (;;) {
        // ---- take the next item from this XCD's queue, then from the others
        if (tid == 0) {
            auto queue_len = [&](int q) {
                return (unsigned int)((ngroups > q ? (ngroups - q + 7) / 8 : 0) * per_group);
            };
            int item = -1;
            while (qi < 8 && item < 0) {
                const int q = (xcc + qi) & 7;
                const unsigned int tk = __hip_atomic_fetch_add(a.tickets + q, 1u, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT);
                if (tk < queue_len(q)) {
                    item = (q + 8 * (int)(tk / per_group)) * per_group + (int)(tk % per_group);
                } else {
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
        const int item = __builtin_amdgcn_readfirstlane(s_item);
        __syncthreads();
        if (item < 0) break;
        // The lane index is made opaque once per item, so that the compiler computes the per-lane
        // addresses of each role inside that role's branch instead of hoisting all of them into
        // the kernel's entry, where they would stay live (and spilled) across every role.
        int lane = tid & 63;
        asm volatile("" : "+v"(lane));
        const int l16 = lane & 15, lq = lane >> 4;
        // item = group * (r NSL) + hr * NSL + s, group = b Hk + kh
        const int grp = item / per_group, wi = item % per_group;
        const int b = grp / a.Hk, kh = grp % a.Hk, hr = wi / NSL, s = wi % NSL;
        const int h = kh * a.r + hr, chain = b * a.Hv + h;
        const SeqInfo si = seq_info(a.cu, b, a.T, a.nch, a.B);
        const int nch = si.nch, sc0 = si.c0;
        const int sv0 = s * BV;
        const int last = nch + 2 + kLagP;
        const size_t qk_stride = (size_t)a.Hk * kQKF, tp_stride = (size_t)a.Hv * kTPF;
        const _Float16 *qk0 = a.qkf + ((size_t)sc0 * a.Hk + kh) * kQKF;
        const _Float16 *tp0 = a.tpf + ((size_t)sc0 * a.Hv + h) * kTPF;
        int broken = 0;

        if (nch == 0) {
            if (tid == 0) atomicOr(a.err, 2u);  // a packed sequence with invalid bounds
        } else if (wave == 0) {
            // ------------------------------------------------------------ state wave
            floatx4 S[NT][8];
            const float *src = a.state_in ? a.state_in + (size_t)chain * kD * kD : nullptr;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int ti = 0; ti < 8; ++ti)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[t][ti][e] = src ? src[(size_t)(16 * ti + 4 * lq + e) * kD + sv0 + 16 * t + l16] : 0.0f;
            half8 fkT[16];
            {
                const __amdgpu_buffer_rsrc_t r0 = make_rsrc(qk0 + kKTOff, 16 * 1024);
#pragma unroll
                for (int f = 0; f < 16; ++f) fkT[f] = ld_frag(r0, lane * 16, f);
            }
            lds_barrier();
            lds_barrier();
            for (int c = 0; c <= last; ++c) {
                if (c < nch) {
                    const __amdgpu_buffer_rsrc_t rn = make_rsrc(qk0 + (size_t)min(c + 1, nch - 1) * qk_stride + kKTOff,
                                                                16 * 1024);
                    state_chunk<NT>(smem, S, fkT, rn, c, lane, l16, lq);
                }
                lds_barrier();
            }
            float *dst = a.state_out + (size_t)chain * kD * kD;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int ti = 0; ti < 8; ++ti)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[(size_t)(16 * ti + 4 * lq + e) * kD + sv0 + 16 * t + l16] = S[t][ti][e];
        } else if (wave == 1) {
            // ------------------------------------------------------------ read-out wave
            half8 fq[16], fp[6];
            float4 eg[4];
            {
                const __amdgpu_buffer_rsrc_t rq = make_rsrc(qk0, 16 * 1024), rt = make_rsrc(tp0, kTPF * 2);
#pragma unroll
                for (int f = 0; f < 16; ++f) fq[f] = ld_frag(rq, lane * 16, f);
#pragma unroll
                for (int f = 0; f < 6; ++f) fp[f] = ld_frag(rt, kPOff * 2 + lane * 16, f);
#pragma unroll
                for (int I = 0; I < 4; ++I) eg[I] = ld_f4(rt, kVecOff * 2 + lq * 16, 64 * I);
            }
            lds_barrier();
            lds_barrier();
            for (int c = 0; c <= last; ++c) {
                if (c >= 1 && c - 1 < nch) {
                    const int cn = min(c, nch - 1);
                    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qk0 + (size_t)cn * qk_stride, 16 * 1024);
                    const __amdgpu_buffer_rsrc_t rt = make_rsrc(tp0 + (size_t)cn * tp_stride, kTPF * 2);
                    readout_chunk<NT>(smem, fq, fp, eg, rq, rt, c - 1, lane, l16, lq);
                }
                lds_barrier();
            }
        } else {
            // ------------------------------------------------------------ helpers
            const int vtid = hidx * 64 + lane;  // 0..383
            // the slice's conv taps and norm weights, and the raw v rows before chunk 0
            if (vtid < BV) {
                const int chn = 2 * a.Hk * kD + h * kD + sv0 + vtid;
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4)
                    sCW[vtid * 4 + t4] = a.conv ? bf16_to_f32(a.conv_w[(size_t)chn * 4 + t4]) : 0.0f;
                sNW[vtid] = a.norm ? bf16_to_f32(a.norm_w[sv0 + vtid]) : 1.0f;
            }
            if (vtid >= 64 && vtid < 64 + 3 * NCG) {
                const int r3 = (vtid - 64) / NCG, cg = (vtid - 64) % NCG;
                uint4 rw = make_uint4(0, 0, 0, 0);
                if (a.conv && a.conv_state_in)
                    rw = *reinterpret_cast<const uint4 *>(a.conv_state_in + ((size_t)b * 3 + r3) * a.Cc + 2 * a.Hk * kD +
                                                          h * kD + sv0 + cg * 8);
                *reinterpret_cast<uint4 *>(sHalo + r3 * BV + cg * 8) = rw;
            }
            // DMA group of chunk cc (helper 1 alone): its k^ fragments and T diag(beta) + decays
            // -> ring slot cc % 3, and (rows_dma) its raw v rows -> ring slot cc % 3.  Chunks past
            // the last repeat the last (a harmless duplicate), so that every iteration issues the
            // same loads.
            const bool dma1 = hidx == 1;
            auto dma_ops = [&](int cc) __attribute__((always_inline)) {
                const int cl = min(cc, nch - 1);
                unsigned char *kslot = smem + L::sK + (cc % 3) * 16384;
                const _Float16 *kb = qk0 + (size_t)cl * qk_stride + kKOff;
#pragma unroll
                for (int f = 0; f < 16; ++f) dma16(kb + f * kFrag + lane * 8, kslot + f * 1024);
                unsigned char *tslot = smem + L::sTB + (cc % 3) * kTB;
                const unsigned char *tb = reinterpret_cast<const unsigned char *>(tp0 + (size_t)cl * tp_stride);
#pragma unroll
                for (int f = 0; f < 7; ++f) dma16(tb + f * 1024 + lane * 16, tslot + f * 1024);
            };
            auto rows_dma = [&](int cc) __attribute__((always_inline)) {
                const int c0 = min(cc, nch - 1) * kC;
                const unsigned int nrow = (unsigned int)min(si.T - c0, kC);
                const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.v + (si.tok0 + c0) * a.Hv * kD, nrow * (unsigned int)a.Hv * kD * 2);
                uint16_t *dst = sRawV + (cc % 3) * kC * BV;
#pragma unroll
                for (int u = 0; u < NRD; ++u) {
                    const int i = lane + 64 * u, row = i / NCG, cg = i % NCG;
                    dma16b(rr, ((row * a.Hv + h) * kD + sv0 + 8 * cg) * 2, dst + u * 512);
                }
            };
            if (dma1) {
                dma_ops(0);
                dma_ops(1);
                rows_dma(0);
                rows_dma(1);
                rows_dma(2);
                wait_vmcnt<0>();
            }
            // conv lane: rows rg * RPI .. +RPI-1, channels 4 c4 .. 4 c4 + 3 of the slice.  Conv
            // slots 0..3 sit on helpers 2..5 (a one-tile slice needs two), never on the DMA
            // helper: the compiler makes every LDS read wait for the DMAs a wave has in flight.
            const int cslot = hidx - 2;
            const int ci = hidx >= 2 && cslot < NCV ? cslot * 64 + lane : -1;
            const int c4 = (ci >= 0 ? ci : 0) % NC4, rg = (ci >= 0 ? ci : 0) / NC4;
            float hwc[16];
            float nw[8];
            // all-ones when the conv / the gated norm is on; opaque to the compiler, which would
            // otherwise turn the selects below back into branches around the transcendentals
            unsigned int conv_mask = a.conv ? ~0u : 0u, norm_mask = a.norm ? ~0u : 0u;
            asm volatile("" : "+v"(conv_mask), "+v"(norm_mask));
            auto conv_v = [&](int cc) __attribute__((always_inline)) {
                if (ci < 0) return;
                const uint16_t *raw = sRawV + (cc % 3) * kC * BV;
                if (ci < 3 * NCG) {  // the chunk's last three raw rows -> halo of the next chunk
                    const int r3 = ci / NCG, cg = ci % NCG;
                    *reinterpret_cast<uint4 *>(sHalo + ((cc + 1) & 1) * 3 * BV + r3 * BV + cg * 8) =
                        *reinterpret_cast<const uint4 *>(raw + (kC - 3 + r3) * BV + cg * 8);
                }
                const int r0 = rg * RPI;
                uint2 rw[RPI + 3];
#pragma unroll
                for (int j = 0; j < RPI + 3; ++j) {
                    const int r2 = r0 - 3 + j;
                    rw[j] = *reinterpret_cast<const uint2 *>(
                        r2 >= 0 ? raw + r2 * BV + c4 * 4 : sHalo + (cc & 1) * 3 * BV + (3 + r2) * BV + c4 * 4);
                }
                float x[RPI + 3][4];
#pragma unroll
                for (int j = 0; j < RPI + 3; ++j) {
                    x[j][0] = __uint_as_float(rw[j].x << 16);
                    x[j][1] = __uint_as_float(rw[j].x & 0xffff0000u);
                    x[j][2] = __uint_as_float(rw[j].y << 16);
                    x[j][3] = __uint_as_float(rw[j].y & 0xffff0000u);
                }
                _Float16 *dst = sV + (cc & 1) * L::SVT + vcol(c4 * 4) + r0;  // columns 4 c4 .. 4 c4 + 3
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float u[RPI];
#pragma unroll
                    for (int i = 0; i < RPI; ++i) {
                        // computed either way and selected: a branch here would split the unrolled
                        // loop into blocks the scheduler cannot interleave
                        const float acc = hwc[4 * e] * x[i][e] + hwc[4 * e + 1] * x[i + 1][e] +
                                          hwc[4 * e + 2] * x[i + 2][e] + hwc[4 * e + 3] * x[i + 3][e];
                        const float sil = acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(acc * -1.4426950408889634f));
                        u[i] = bit_select(conv_mask, sil, x[i + 3][e]);
                    }
                    *reinterpret_cast<halfx2 *>(dst + e * kVStride) = halfx2{static_cast<_Float16>(u[0]), static_cast<_Float16>(u[1])};
                }
            };
            lds_barrier();  // taps, weights and halo staged; DMA groups 0, 1 landed
#pragma unroll
            for (int e = 0; e < 16; ++e) hwc[e] = sCW[c4 * 16 + e];
            conv_v(0);
            lds_barrier();

            if (hidx == 0) {
                // ---------------------------------------------- norm exchange (no DMA, no stores but the mailbox)
                // One counter tracks this wave's loads and stores in issue order, so every load and
                // store here is issued unconditionally and in a fixed order, and the sibling words
                // for the next iteration are requested before this iteration's publish: waiting for
                // them then never waits for a store.  Two register sets alternate between iterations.
                unsigned long long *mrow = a.mbox + (size_t)chain * kTiles * kMboxRing * kC + lane;  // row = lane
                unsigned long long *trash = a.mbox + (size_t)a.B * a.Hv * kTiles * kMboxRing * kC + lane;
                unsigned long long mA[NSL], mB[NSL];
                int xrow[NCG];  // position of row `lane` in each 8-column group's columns
#pragma unroll
                for (int g = 0; g < NCG; ++g) xrow[g] = orow(BV, lane, 8 * g);
                auto mb_request = [&](int cc, unsigned long long(&m)[NSL]) __attribute__((always_inline)) {
                    const int ccl = min(max(cc, 0), nch - 1);
#pragma unroll
                    for (int sib = 0; sib < NSL; ++sib)
                        m[sib] = __hip_atomic_load(mrow + ((size_t)sib * kMboxRing + (ccl % kMboxRing)) * kC, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                };
                auto step = [&](int c, unsigned long long(&mcur)[NSL], unsigned long long(&mnext)[NSL])
                                __attribute__((always_inline)) {
                    const int rc = c - 2 - kLagP;
                    mb_request(rc + 1, mnext);
                    // 1/rms of chunk rc from every slice's words (a word without the chunk's tag is waited for)
                    if (a.norm && rc >= 0 && rc < nch) {
                        float tot = 0.0f;
#pragma unroll
                        for (int sib = 0; sib < NSL; ++sib) {
                            unsigned long long w = mcur[sib];
                            if ((uint32_t)(w >> 32) != (uint32_t)(rc + 1))
                                w = spin_load(mrow + ((size_t)sib * kMboxRing + (rc % kMboxRing)) * kC, (uint32_t)(rc + 1), a.err,
                                              broken);
                            tot += __uint_as_float((uint32_t)w);
                        }
                        // a timed-out wait leaves the rows NaN rather than quietly wrong
                        sRstd[(rc & 1) * kC + lane] =
                            broken ? __builtin_nanf("") : __builtin_amdgcn_rsqf(tot * (1.0f / kD) + a.eps_norm);
                    }
                    // row sums of chunk c - 2 over this slice's columns -> mailbox (tag c - 1); outside
                    // the chunk range the word goes to a scratch row nobody reads
                    const bool pub = c >= 2 && c - 2 < nch;
                    const float *src = sO + ((pub ? c - 2 : 0) % kORingP) * VT;
                    float ss = 0.0f;
#pragma unroll
                    for (int j = 0; j < BV; ++j) {
                        const float x = src[j * PL + xrow[j >> 3]];
                        ss += x * x;
                    }
                    __hip_atomic_store(pub ? mrow + ((size_t)s * kMboxRing + ((c - 2) % kMboxRing)) * kC : trash,
                                       ((unsigned long long)(uint32_t)(c - 1) << 32) | __float_as_uint(ss),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    lds_barrier();
                };
                mb_request(-2 - kLagP, mA);
                int c = 0;
                for (; c + 1 <= last; c += 2) {
                    step(c, mA, mB);
                    step(c + 1, mB, mA);
                }
                if (c <= last) step(c, mA, mB);
            } else if (dma1) {
                // ---------------------------------------------- DMA only
                for (int c = 0; c <= last; ++c) {
                    __builtin_amdgcn_sched_barrier(0);
                    dma_ops(c + 2);
                    rows_dma(c + 3);
                    // the previous iteration's group has landed
                    wait_vmcnt<16 + 7 + NRD>();
                    __builtin_amdgcn_s_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
                }
                wait_vmcnt<0>();
            } else {
                // ---------------------------------------------- conv (if any) and gating + store
                const int gl = (hidx - (6 - NGT)) * 64 + lane;  // gating lane 0 .. 64 NGT - 1
                static_assert(NGT == 4, "helpers 2, 3, 4, 5 all gate");
                int cg8[GPL];
#pragma unroll
                for (int u = 0; u < GPL; ++u) cg8[u] = ((gl + 64 * NGT * u) % NCG);
#pragma unroll
                for (int e = 0; e < 8; ++e) nw[e] = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) nw[e] = sNW[cg8[0] * 8 + e];  // GPL items share the column group
                // z rows of chunk oc for this lane's items, through a buffer resource over the chunk's
                // rows (rows past T read as zero).  Loads and stores are unconditional and in a fixed
                // order (the next chunk's z is requested before this chunk's stores), for the same
                // reason as in the exchange helper; outside the chunk range the stores go to a
                // zero-sized resource and are dropped.
                const uint16_t *zsrc = a.norm ? a.z : a.v;
                auto rows_rsrc = [&](const uint16_t *base, int oc) __attribute__((always_inline)) {
                    const int ocl = min(max(oc, 0), nch - 1);
                    const unsigned int nrow = (oc >= 0 && oc < nch) ? (unsigned int)min(si.T - ocl * kC, kC) : 0u;
                    return make_rsrc(base + (si.tok0 + (size_t)ocl * kC) * a.Hv * kD, nrow * (unsigned int)a.Hv * kD * 2);
                };
                int voff[GPL], grow[GPL];  // grow: the item's row position in its columns of sO
#pragma unroll
                for (int u = 0; u < GPL; ++u) {
                    const int it = gl + 64 * NGT * u, row = it < NGATE ? it / NCG : kC;  // row kC: past every resource
                    voff[u] = ((row * a.Hv + h) * kD + sv0 + cg8[u] * 8) * 2;
                    grow[u] = orow(BV, it < NGATE ? row : 0, 8 * cg8[u]);
                }
                auto z_load = [&](int oc, uint4(&z)[GPL]) __attribute__((always_inline)) {
                    const __amdgpu_buffer_rsrc_t rz = rows_rsrc(zsrc, oc);
#pragma unroll
                    for (int u = 0; u < GPL; ++u)
                        z[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rz, voff[u], 0, 0));
                };
                auto step = [&](int c, uint4(&zcur)[GPL], uint4(&znext)[GPL]) __attribute__((always_inline)) {
                    const int oc = c - 3 - kLagP;
                    z_load(oc + 1, znext);
                    if (c + 1 < nch) conv_v(c + 1);
                    {
                        const int ocl = max(oc, 0);
                        const float *src = sO + (ocl % kORingP) * VT;
                        const float *rs = sRstd + (ocl & 1) * kC;
                        const __amdgpu_buffer_rsrc_t ro = rows_rsrc(a.o, oc);
#pragma unroll
                        for (int u = 0; u < GPL; ++u) {
                            const int it = gl + 64 * NGT * u, row = (it < NGATE ? it : 0) / NCG;
                            float y[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) y[e] = src[(cg8[u] * 8 + e) * PL + grow[u]];
                            // the gated norm is computed either way and selected (no branch in the
                            // unrolled loop; without the norm z is the readable v and rstd unused)
                            float zf[8];
                            unpack_bf16x8(zcur[u], zf);
                            const float rstd = rs[row];
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(zf[e] * -1.4426950408889634f));
                                const float yn = nw[e] * (y[e] * rstd) * (zf[e] * sg);
                                y[e] = bit_select(norm_mask, yn, y[e]);
                            }
                            const uint4 pk = pack_bf16x8(y);
                            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pk.x, pk.y, pk.z, pk.w}, ro, voff[u], 0, 0);
                        }
                    }
                    lds_barrier();
                };
                uint4 zA[GPL], zB[GPL];
                z_load(-3 - kLagP, zA);
                int c = 0;
                for (; c + 1 <= last; c += 2) {
                    step(c, zA, zB);
                    step(c + 1, zB, zA);
                }
                if (c <= last) step(c, zA, zB);
            }
            // raw v inputs of the last three tokens -> conv state out (v channels of this slice)
            if (hidx == 0 && a.conv && a.conv_state_out && lane < 3 * NCG) {
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
        __syncthreads();
    }
}

} // namespace

// Launch shape of the sequential pass for this device (resident slots queried once per
// device and tile count).
struct PassFacts {
    int ncu = 0;
    int per_cu[2] = {0, 0};
};

int launch_pass(const PrefillParams &p, const PrefillPlan &plan, const PrefillRegions &rg, hipStream_t stream) {
    static PassFacts facts[64];
    static std::mutex mu;
    int dev = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return fail("hipGetDevice", e);
    if (dev < 0 || dev >= 64) return fail("prefill: device index out of range");
    const int nt = plan.nt;
    const void *fn = nt == 1 ? reinterpret_cast<const void *>(pass_kernel<1>) : reinterpret_cast<const void *>(pass_kernel<2>);
    const size_t lds = nt == 1 ? PassLds<1>::bytes : PassLds<2>::bytes;
    int ncu, per_cu;
    {
        std::lock_guard<std::mutex> g(mu);
        PassFacts &f = facts[dev];
        if (!f.ncu && (e = hipDeviceGetAttribute(&f.ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
            return fail("hipDeviceGetAttribute(multiprocessor count)", e);
        int &pc = f.per_cu[nt - 1];
        if (!pc) {
            if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
                return fail("hipFuncSetAttribute(pass_kernel)", e);
            if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, fn, 512, lds)) != hipSuccess)
                return fail("hipOccupancyMaxActiveBlocksPerMultiprocessor(pass_kernel)", e);
            if (pc < 1) return fail("pass_kernel: no resident workgroup fits a compute unit");
        }
        ncu = f.ncu;
        per_cu = pc;
    }
    const int nsl = kTiles / nt;
    const long long items = (long long)p.B * p.Hv * nsl;
    // A workgroup that waits for its sibling slices holds its slot, and the ticket order
    // lets the next free slot start them; the slices of one head are consecutive tickets
    // of one queue, so every queue needs room for one head's slices.
    const int cap = ncu * per_cu;
    if (cap < 8 * nsl) return fail("pass_kernel: fewer resident workgroup slots than eight heads' slices");
    const int grid = (int)std::min<long long>(items, cap);

    PassArgs a;
    a.qkf = rg.qkf; a.tpf = rg.tpf;
    a.v = p.v; a.z = p.z; a.conv_w = p.conv_w; a.norm_w = p.norm_w; a.conv_state_in = p.conv_state_in;
    a.state_in = p.state_in; a.o = p.o; a.conv_state_out = p.conv_state_out; a.state_out = p.state_out;
    a.mbox = rg.mbox; a.err = rg.err; a.tickets = rg.tickets; a.cu = p.cu_seqlens;
    a.B = p.B; a.T = p.T; a.Hk = p.Hk; a.Hv = p.Hv; a.r = p.Hv / p.Hk; a.Cc = 2 * p.Hk * kD + p.Hv * kD;
    a.conv = p.conv_width == 4; a.norm = p.norm; a.nch = plan.nchunks; a.eps_norm = p.eps_norm;
    void *args[] = {&a};
    if ((e = hipLaunchKernel(fn, dim3(grid), dim3(512), args, lds, stream)) != hipSuccess)
        return fail("hipLaunchKernel(pass_kernel)", e);
    return 0;
}

} // namespace gdn
